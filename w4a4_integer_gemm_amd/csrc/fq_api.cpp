// C ABI of libfq: argument validation, error messages and kernel dispatch.
//
// Every check runs before any HIP call, so a rejected call queues no device
// work and writes nothing.  The messages follow the page's convention of
// naming the call and argument and showing the arithmetic that failed.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>

#include "../../include/fq.h"
#include "fq_internal.h"

namespace fq {

static thread_local std::string g_error;

void set_error(const std::string& msg) { g_error = msg; }
void clear_error() { g_error.clear(); }

namespace {

// Applies a test-hook spec "key=value,key=value" (keys gemm_tile, gemm_mfma,
// gemv, decode1; "" or "default" resets every hook).  Returns false, with the reason in
// *why, on an unknown key or value; nothing changes then.
bool apply_hooks(Hooks& h, const char* spec, std::string* why) {
    int tile = -1, mfma = 16, split = 0, d1off = 0;
    std::string s = spec ? spec : "";
    if (s == "default") s.clear();
    size_t pos = 0;
    while (pos < s.size()) {
        size_t end = s.find(',', pos);
        if (end == std::string::npos) end = s.size();
        const std::string item = s.substr(pos, end - pos);
        pos = end + 1;
        if (item.empty()) continue;
        const size_t eq = item.find('=');
        const std::string key = item.substr(0, eq), val = eq == std::string::npos ? "" : item.substr(eq + 1);
        if (key == "gemm_tile") {
            tile = val == "auto" ? -1 : gemm_tile_id(val.c_str());
            if (tile < 0 && val != "auto") {
                *why = "unknown gemm_tile '" + val + "'";
                return false;
            }
        } else if (key == "gemm_mfma") {
            if (val != "16" && val != "32") {
                *why = "gemm_mfma must be 16 or 32, not '" + val + "'";
                return false;
            }
            mfma = val == "16" ? 16 : 32;
        } else if (key == "gemv") {
            if (val != "split" && val != "auto") {
                *why = "gemv must be split or auto, not '" + val + "'";
                return false;
            }
            split = val == "split";
        } else if (key == "decode1") {
            if (val != "off" && val != "auto") {
                *why = "decode1 must be off or auto, not '" + val + "'";
                return false;
            }
            d1off = val == "off";
        } else {
            *why = "unknown hook '" + key + "' (gemm_tile, gemm_mfma, gemv, decode1)";
            return false;
        }
    }
    h.gemm_tile.store(tile, std::memory_order_relaxed);
    h.gemm_mfma.store(mfma, std::memory_order_relaxed);
    h.gemv_split.store(split, std::memory_order_relaxed);
    h.decode1_off.store(d1off, std::memory_order_relaxed);
    return true;
}

Hooks* make_hooks() {
    static Hooks h;
    std::string why;
    const char* env = std::getenv("FQ_TEST_HOOK");  // read once per process
    if (env && !apply_hooks(h, env, &why)) std::fprintf(stderr, "libfq: FQ_TEST_HOOK ignored: %s\n", why.c_str());
    return &h;
}

DeviceInfo g_devices[kMaxDevices];
hipError_t g_device_err[kMaxDevices];
std::once_flag g_device_once[kMaxDevices];

hipError_t init_device(int dev, DeviceInfo& d) {
    d.device = dev;
    hipError_t e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&d.lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e == hipSuccess && (d.cus < 1 || d.lds_per_cu < 1)) e = hipErrorInvalidDevice;
    if (e == hipSuccess) e = init_gemv_device(d);
    if (e == hipSuccess) e = init_scratch_device(d);
    return e;
}

}  // namespace

Hooks& hooks() {
    static Hooks* const h = make_hooks();
    return *h;
}

hipError_t prepare_device(const DeviceInfo** info) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_device_once[dev], [dev] { g_device_err[dev] = init_device(dev, g_devices[dev]); });
    if (g_device_err[dev] != hipSuccess) return g_device_err[dev];
    *info = &g_devices[dev];
    return hipSuccess;
}

}  // namespace fq

namespace {

std::string fmt(const char* f, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, f);
    vsnprintf(buf, sizeof(buf), f, ap);
    va_end(ap);
    return std::string(buf);
}

fq_status fail(fq_status s, const std::string& msg) {
    fq::set_error(msg);
    return s;
}

bool is_pow2(int64_t v) { return v >= 1 && (v & (v - 1)) == 0; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int32_t kMaxK = 65536;
constexpr int32_t kProloguePack = 32;  // 32 bf16 values per prologue lane
constexpr int32_t kGemmK = 128;        // one k stage of the GEMM

// Checks shared by the prologue, the GEMM and the packer.  Returns FQ_OK or the failure.
fq_status check_bits(const char* fn, const char* name, int32_t bits) {
    if (bits != 8 && bits != 4 && bits != FQ_CODES_E2M3)
        return fail(FQ_ERR_UNSUPPORTED,
                    fmt("%s: %s=%d is not a supported code width (4, 8, or 6 for E2M3)", fn, name, bits));
    return FQ_OK;
}

// K bounds; `mult` is the granularity the entry point needs (32 for the
// prologue, whose lanes hold up to 32 values each below K = 32768; 128 for the
// GEMM's k stages).
fq_status check_k(const char* fn, int32_t K, int32_t mult) {
    if (K < mult || K > kMaxK)
        return fail(FQ_ERR_SHAPE, fmt("%s: K=%d outside [%d, %d]", fn, K, mult, kMaxK));
    if (K % mult)
        return fail(FQ_ERR_SHAPE, fmt("%s: K=%d is not a multiple of %d (%d/%d = %.2f)", fn, K, mult, K, mult,
                                      double(K) / mult));
    return FQ_OK;
}

fq_status check_hblock(const char* fn, int32_t K, int32_t hblock) {
    if (!is_pow2(hblock) || hblock > 256)
        return fail(FQ_ERR_SHAPE, fmt("%s: hblock=%d must be a power of two in [1, 256]", fn, hblock));
    if (K % hblock)
        return fail(FQ_ERR_SHAPE, fmt("%s: K=%d not divisible by hblock=%d (%d/%d = %.2f)", fn, K, hblock,
                                      K, hblock, double(K) / hblock));
    return FQ_OK;
}

#define FQ_TRY(expr)                     \
    do {                                 \
        fq_status _s = (expr);           \
        if (_s != FQ_OK) return _s;      \
    } while (0)

fq_status validate_prologue(const char* fn, const void* x, int32_t M, int32_t K, int64_t ldx,
                            const float* gamma, float eps, const float* ascale, int32_t fold_after,
                            int32_t hblock, int32_t abits, const void* codes, const float* scale,
                            bool check_out = true) {
    if (!x) return fail(FQ_ERR_ARG, fmt("%s: x_bf16 is NULL", fn));
    if (check_out && !codes) return fail(FQ_ERR_ARG, fmt("%s: act_codes is NULL", fn));
    if (check_out && !scale) return fail(FQ_ERR_ARG, fmt("%s: act_scale is NULL", fn));
    if (M < 1) return fail(FQ_ERR_SHAPE, fmt("%s: M=%d must be >= 1", fn, M));
    FQ_TRY(check_k(fn, K, kProloguePack));
    if (K > 32768 && K % 64)
        return fail(FQ_ERR_SHAPE, fmt("%s: K=%d above 32768 must be a multiple of 64 (%d/64 = %.2f)", fn, K, K,
                                      K / 64.0));
    FQ_TRY(check_bits(fn, "abits", abits));
    FQ_TRY(check_hblock(fn, K, hblock));
    if (ldx < K) return fail(FQ_ERR_SHAPE, fmt("%s: ldx=%lld < K=%d", fn, (long long)ldx, K));
    if (ldx % 8) return fail(FQ_ERR_ALIGN, fmt("%s: ldx=%lld is not a multiple of 8 bf16 (16 bytes)", fn, (long long)ldx));
    if (fold_after != 0 && fold_after != 1)
        return fail(FQ_ERR_ARG, fmt("%s: fold_after=%d must be 0 or 1", fn, fold_after));
    if (gamma && !(eps >= 0.0f && eps < 1e30f))
        return fail(FQ_ERR_ARG, fmt("%s: eps=%g must be finite and >= 0", fn, (double)eps));
    if (!aligned(x, 16)) return fail(FQ_ERR_ALIGN, fmt("%s: x_bf16 is not 16-byte aligned", fn));
    if (check_out && !aligned(codes, 16)) return fail(FQ_ERR_ALIGN, fmt("%s: act_codes is not 16-byte aligned", fn));
    if (check_out && !aligned(scale, 4)) return fail(FQ_ERR_ALIGN, fmt("%s: act_scale is not 4-byte aligned", fn));
    if (gamma && !aligned(gamma, 16)) return fail(FQ_ERR_ALIGN, fmt("%s: gamma_folded is not 16-byte aligned", fn));
    if (ascale && !aligned(ascale, 16)) return fail(FQ_ERR_ALIGN, fmt("%s: ascale is not 16-byte aligned", fn));
    return FQ_OK;
}

fq_status validate_gemm(const char* fn, const void* act, const float* act_scale, int32_t M, int32_t abits,
                        const void* w, const float* wscale, int32_t N, int32_t K, int32_t wbits,
                        const float* bias, const void* residual, int64_t ldr, const void* y, int64_t ldy,
                        bool check_act, int32_t head_dim = 0) {
    if (check_act && !act) return fail(FQ_ERR_ARG, fmt("%s: act_codes is NULL", fn));
    if (check_act && !act_scale) return fail(FQ_ERR_ARG, fmt("%s: act_scale is NULL", fn));
    if (!w) return fail(FQ_ERR_ARG, fmt("%s: w_codes is NULL", fn));
    if (!wscale) return fail(FQ_ERR_ARG, fmt("%s: wscale is NULL", fn));
    if (!y) return fail(FQ_ERR_ARG, fmt("%s: y_bf16 is NULL", fn));
    if (M < 1) return fail(FQ_ERR_SHAPE, fmt("%s: M=%d must be >= 1", fn, M));
    if (N < 1) return fail(FQ_ERR_SHAPE, fmt("%s: N=%d must be >= 1", fn, N));
    if (N % 8) return fail(FQ_ERR_SHAPE, fmt("%s: N=%d is not a multiple of 8 (%d/8 = %.3f)", fn, N, N, N / 8.0));
    FQ_TRY(check_k(fn, K, kGemmK));
    FQ_TRY(check_bits(fn, "abits", abits));
    FQ_TRY(check_bits(fn, "wbits", wbits));
    if ((abits == FQ_CODES_E2M3) != (wbits == FQ_CODES_E2M3))
        return fail(FQ_ERR_UNSUPPORTED, fmt("%s: abits=%d with wbits=%d: E2M3 codes (6) need both operands in E2M3",
                                            fn, abits, wbits));
    if (head_dim > 0) {
        if (head_dim % 8)
            return fail(FQ_ERR_SHAPE, fmt("%s: head_dim=%d is not a multiple of 8", fn, head_dim));
        if (N % head_dim)
            return fail(FQ_ERR_SHAPE, fmt("%s: N=%d is not a whole number of heads of head_dim=%d (%d/%d = %.3f)", fn,
                                          N, head_dim, N, head_dim, double(N) / head_dim));
    } else if (head_dim < 0) {
        return fail(FQ_ERR_SHAPE, fmt("%s: head_dim=%d must be > 0", fn, head_dim));
    } else {
        if (ldy < N) return fail(FQ_ERR_SHAPE, fmt("%s: ldy=%lld < N=%d", fn, (long long)ldy, N));
        if (ldy % 8) return fail(FQ_ERR_ALIGN, fmt("%s: ldy=%lld is not a multiple of 8 bf16", fn, (long long)ldy));
    }
    if (residual && ldr < N) return fail(FQ_ERR_SHAPE, fmt("%s: ldr=%lld < N=%d", fn, (long long)ldr, N));
    if (residual && ldr % 8) return fail(FQ_ERR_ALIGN, fmt("%s: ldr=%lld is not a multiple of 8 bf16", fn, (long long)ldr));
    if (check_act && !aligned(act, 16)) return fail(FQ_ERR_ALIGN, fmt("%s: act_codes is not 16-byte aligned", fn));
    if (check_act && !aligned(act_scale, 4)) return fail(FQ_ERR_ALIGN, fmt("%s: act_scale is not 4-byte aligned", fn));
    if (!aligned(w, 16)) return fail(FQ_ERR_ALIGN, fmt("%s: w_codes is not 16-byte aligned", fn));
    if (!aligned(wscale, 16)) return fail(FQ_ERR_ALIGN, fmt("%s: wscale is not 16-byte aligned", fn));
    if (bias && !aligned(bias, 16)) return fail(FQ_ERR_ALIGN, fmt("%s: bias is not 16-byte aligned", fn));
    if (residual && !aligned(residual, 16)) return fail(FQ_ERR_ALIGN, fmt("%s: residual_bf16 is not 16-byte aligned", fn));
    if (!aligned(y, 16)) return fail(FQ_ERR_ALIGN, fmt("%s: y_bf16 is not 16-byte aligned", fn));
    return FQ_OK;
}

fq_status device_status(const char* fn, hipError_t e) {
    if (e != hipSuccess) return fail(FQ_ERR_DEVICE, fmt("%s: %s", fn, hipGetErrorString(e)));
    return FQ_OK;
}

size_t code_bytes(int32_t rows, int32_t K, int32_t bits) {
    if (rows < 1 || K < 4 || K % 4 || (bits != 4 && bits != 8 && bits != FQ_CODES_E2M3)) return 0;
    if (bits == FQ_CODES_E2M3) return size_t(rows) * size_t(3 * (K / 4));
    return bits == 8 ? size_t(rows) * size_t(K) : size_t(rows) * size_t(K / 2);
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// The device set-up every device entry point runs before it queues anything.
fq_status prepare(const char* fn, const fq::DeviceInfo** info) {
    return device_status(fn, fq::prepare_device(info));
}

fq_status run_gemm(const char* fn, const fq::GemmArgs& g, const fq::DeviceInfo& dev, hipStream_t stream) {
    hipError_t e = g.abits == FQ_CODES_E2M3   ? fq::launch_gemm_e2m3(g, stream)
                   : g.M <= fq::kGemvMaxM ? fq::launch_gemv(g, dev, stream)
                                          : fq::launch_gemm(g, stream);
    return device_status(fn, e);
}

}  // namespace

extern "C" {

const char* fq_last_error(void) { return fq::g_error.c_str(); }

int fq_abi_version(void) { return FQ_ABI_VERSION; }

size_t fq_weight_bytes(int32_t N, int32_t K, int32_t wbits) { return code_bytes(N, K, wbits); }

size_t fq_act_bytes(int32_t M, int32_t K, int32_t abits) { return code_bytes(M, K, abits); }

size_t fq_linear_workspace_bytes(int32_t M, int32_t K, int32_t abits) {
    size_t c = code_bytes(M, K, abits);
    if (!c) return 0;
    return round_up(c, 256) + round_up(size_t(M) * sizeof(float), 256);
}

fq_status fq_fold_gain(const float* gamma, const float* ascale, int32_t K, float* gamma_out) {
    fq::clear_error();
    if (!gamma || !gamma_out) return fail(FQ_ERR_ARG, "fq_fold_gain: gamma or gamma_out is NULL");
    if (K < 1) return fail(FQ_ERR_SHAPE, fmt("fq_fold_gain: K=%d must be >= 1", K));
    if (ascale) {
        for (int32_t k = 0; k < K; ++k)
            if (!(ascale[k] > 0.0f))
                return fail(FQ_ERR_ARG, fmt("fq_fold_gain: ascale[%d]=%g must be > 0", k, (double)ascale[k]));
    }
    for (int32_t k = 0; k < K; ++k) gamma_out[k] = ascale ? gamma[k] / ascale[k] : gamma[k];
    return FQ_OK;
}

fq_status fq_prologue(const void* x_bf16, int32_t M, int32_t K, int64_t ldx, const float* gamma_folded,
                      float eps, const float* ascale, int32_t fold_after, int32_t hblock, int32_t abits,
                      void* act_codes, float* act_scale, void* stream) {
    fq::clear_error();
    const char* fn = "fq_prologue";
    FQ_TRY(validate_prologue(fn, x_bf16, M, K, ldx, gamma_folded, eps, ascale, fold_after, hblock, abits,
                             act_codes, act_scale));
    const fq::DeviceInfo* dev = nullptr;
    FQ_TRY(prepare(fn, &dev));
    fq::PrologueArgs a{static_cast<const uint16_t*>(x_bf16), M, K, ldx, gamma_folded, eps, ascale,
                       fold_after, hblock, abits, static_cast<uint8_t*>(act_codes), act_scale};
    return device_status(fn, fq::launch_prologue(a, static_cast<hipStream_t>(stream)));
}

fq_status fq_device_init(void) {
    fq::clear_error();
    const fq::DeviceInfo* dev = nullptr;
    return prepare("fq_device_init", &dev);
}

fq_status fq_test_hook(const char* spec) {
    fq::clear_error();
    std::string why;
    if (!fq::apply_hooks(fq::hooks(), spec, &why)) return fail(FQ_ERR_ARG, "fq_test_hook: " + why);
    return FQ_OK;
}

}  // extern "C"

namespace {

fq_status gemm_impl(const char* fn, const void* act_codes, const float* act_scale, int32_t M, int32_t abits,
                    const void* w_codes, const float* wscale, int32_t N, int32_t K, int32_t wbits, const float* bias,
                    const void* residual_bf16, int64_t ldr, void* y_bf16, int64_t ldy, int32_t head_dim,
                    int32_t* acc_i32, void* stream) {
    fq::clear_error();
    FQ_TRY(validate_gemm(fn, act_codes, act_scale, M, abits, w_codes, wscale, N, K, wbits, bias, residual_bf16,
                         ldr, y_bf16, ldy, true, head_dim));
    if (acc_i32 && !aligned(acc_i32, 16)) return fail(FQ_ERR_ALIGN, fmt("%s: acc_i32 is not 16-byte aligned", fn));
    const fq::DeviceInfo* dev = nullptr;
    FQ_TRY(prepare(fn, &dev));
    fq::GemmArgs g{static_cast<const uint8_t*>(act_codes), act_scale, M, abits,
                   static_cast<const uint8_t*>(w_codes), wscale, N, K, wbits, bias,
                   static_cast<const uint16_t*>(residual_bf16), ldr, static_cast<uint16_t*>(y_bf16), ldy,
                   acc_i32, head_dim};
    return run_gemm(fn, g, *dev, static_cast<hipStream_t>(stream));
}

// fq_linear and its variants.  With use_scratch the workspace is this
// device's scratch array (fq_linear_noalloc) and workspace/workspace_bytes
// are ignored.
fq_status linear_impl(const char* fn, const void* x_bf16, int32_t M, int32_t K, int64_t ldx,
                      const float* gamma_folded, float eps, const float* ascale, int32_t fold_after, int32_t hblock,
                      int32_t abits, const void* w_codes, const float* wscale, int32_t N, int32_t wbits,
                      const float* bias, const void* residual_bf16, int64_t ldr, void* y_bf16, int64_t ldy,
                      int32_t head_dim, void* workspace, size_t workspace_bytes, void* stream,
                      bool use_scratch = false) {
    fq::clear_error();
    if (!use_scratch && !workspace) return fail(FQ_ERR_ARG, fmt("%s: workspace is NULL", fn));
    if (!use_scratch && !aligned(workspace, 256))
        return fail(FQ_ERR_ALIGN, fmt("%s: workspace is not 256-byte aligned", fn));
    // shape checks first so that the workspace size below is meaningful
    if (M < 1) return fail(FQ_ERR_SHAPE, fmt("%s: M=%d must be >= 1", fn, M));
    FQ_TRY(check_k(fn, K, kGemmK));
    FQ_TRY(check_bits(fn, "abits", abits));
    const size_t need = fq_linear_workspace_bytes(M, K, abits);
    if (use_scratch) {
        if (need > fq::kNoallocScratchBytes)
            return fail(FQ_ERR_UNSUPPORTED,
                        fmt("%s: M=%d K=%d abits=%d needs %zu bytes of codes and scales, more than the %zu-byte "
                            "scratch array; use fq_linear with a caller workspace",
                            fn, M, K, abits, need, fq::kNoallocScratchBytes));
    } else if (workspace_bytes < need) {
        return fail(FQ_ERR_ARG, fmt("%s: workspace_bytes=%zu < %zu needed for M=%d K=%d abits=%d", fn,
                                    workspace_bytes, need, M, K, abits));
    }
    // the device set-up (which also gives this device's scratch address) is
    // the last host-side step that can fail; it runs before anything is queued
    const fq::DeviceInfo* dev = nullptr;
    if (use_scratch) {
        // validate everything that does not depend on the workspace address first
        FQ_TRY(validate_prologue(fn, x_bf16, M, K, ldx, gamma_folded, eps, ascale, fold_after, hblock, abits,
                                 nullptr, nullptr, false));
        FQ_TRY(validate_gemm(fn, nullptr, nullptr, M, abits, w_codes, wscale, N, K, wbits, bias, residual_bf16, ldr,
                             y_bf16, ldy, false, head_dim));
        FQ_TRY(prepare(fn, &dev));
        workspace = dev->scratch;
    }
    uint8_t* codes = static_cast<uint8_t*>(workspace);
    float* scales = reinterpret_cast<float*>(codes + round_up(code_bytes(M, K, abits), 256));
    FQ_TRY(validate_prologue(fn, x_bf16, M, K, ldx, gamma_folded, eps, ascale, fold_after, hblock, abits, codes,
                             scales));
    FQ_TRY(validate_gemm(fn, codes, scales, M, abits, w_codes, wscale, N, K, wbits, bias, residual_bf16, ldr,
                         y_bf16, ldy, true, head_dim));
    if (!use_scratch) FQ_TRY(prepare(fn, &dev));
    hipStream_t s = static_cast<hipStream_t>(stream);
    fq::PrologueArgs a{static_cast<const uint16_t*>(x_bf16), M, K, ldx, gamma_folded, eps, ascale,
                       fold_after, hblock, abits, codes, scales};
    fq::GemmArgs g{codes, scales, M, abits, static_cast<const uint8_t*>(w_codes), wscale, N, K, wbits, bias,
                   static_cast<const uint16_t*>(residual_bf16), ldr, static_cast<uint16_t*>(y_bf16), ldy,
                   nullptr, head_dim};
    // one token: prologue and GEMV in one launch (the same codes, scale and outputs)
    if (fq::decode1_eligible(a, g)) return device_status(fn, fq::launch_decode1(a, g, s));
    FQ_TRY(device_status(fn, fq::launch_prologue(a, s)));
    return run_gemm(fn, g, *dev, s);
}

}  // namespace

extern "C" {

fq_status fq_gemm(const void* act_codes, const float* act_scale, int32_t M, int32_t abits, const void* w_codes,
                  const float* wscale, int32_t N, int32_t K, int32_t wbits, const float* bias,
                  const void* residual_bf16, int64_t ldr, void* y_bf16, int64_t ldy, int32_t* acc_i32,
                  void* stream) {
    return gemm_impl("fq_gemm", act_codes, act_scale, M, abits, w_codes, wscale, N, K, wbits, bias, residual_bf16,
                     ldr, y_bf16, ldy, 0, acc_i32, stream);
}

fq_status fq_gemm_heads(const void* act_codes, const float* act_scale, int32_t M, int32_t abits,
                        const void* w_codes, const float* wscale, int32_t N, int32_t K, int32_t wbits,
                        const float* bias, const void* residual_bf16, int64_t ldr, int32_t head_dim, void* y_bf16,
                        int32_t* acc_i32, void* stream) {
    return gemm_impl("fq_gemm_heads", act_codes, act_scale, M, abits, w_codes, wscale, N, K, wbits, bias,
                     residual_bf16, ldr, y_bf16, 0, head_dim, acc_i32, stream);
}

fq_status fq_linear(const void* x_bf16, int32_t M, int32_t K, int64_t ldx, const float* gamma_folded, float eps,
                    const float* ascale, int32_t fold_after, int32_t hblock, int32_t abits, const void* w_codes,
                    const float* wscale, int32_t N, int32_t wbits, const float* bias, const void* residual_bf16,
                    int64_t ldr, void* y_bf16, int64_t ldy, void* workspace, size_t workspace_bytes,
                    void* stream) {
    return linear_impl("fq_linear", x_bf16, M, K, ldx, gamma_folded, eps, ascale, fold_after, hblock, abits,
                       w_codes, wscale, N, wbits, bias, residual_bf16, ldr, y_bf16, ldy, 0, workspace,
                       workspace_bytes, stream);
}

fq_status fq_geglu(const void* gateup_bf16, int32_t M, int32_t F, int64_t ld_in, void* h_bf16, int64_t ld_out,
                   void* stream) {
    fq::clear_error();
    const char* fn = "fq_geglu";
    if (!gateup_bf16) return fail(FQ_ERR_ARG, "fq_geglu: gateup_bf16 is NULL");
    if (!h_bf16) return fail(FQ_ERR_ARG, "fq_geglu: h_bf16 is NULL");
    if (M < 1) return fail(FQ_ERR_SHAPE, fmt("%s: M=%d must be >= 1", fn, M));
    if (F < 8 || F % 8) return fail(FQ_ERR_SHAPE, fmt("%s: F=%d must be a positive multiple of 8", fn, F));
    if (int64_t(M) * (F / 8) > int64_t(INT32_MAX) * 256)
        return fail(FQ_ERR_SHAPE, fmt("%s: M=%d x F=%d is too large for one launch", fn, M, F));
    if (ld_in < 2 * int64_t(F))
        return fail(FQ_ERR_SHAPE, fmt("%s: ld_in=%lld < 2F=%lld", fn, (long long)ld_in, 2 * (long long)F));
    if (ld_in % 8) return fail(FQ_ERR_ALIGN, fmt("%s: ld_in=%lld is not a multiple of 8 bf16", fn, (long long)ld_in));
    if (ld_out < F) return fail(FQ_ERR_SHAPE, fmt("%s: ld_out=%lld < F=%d", fn, (long long)ld_out, F));
    if (ld_out % 8) return fail(FQ_ERR_ALIGN, fmt("%s: ld_out=%lld is not a multiple of 8 bf16", fn, (long long)ld_out));
    if (!aligned(gateup_bf16, 16)) return fail(FQ_ERR_ALIGN, "fq_geglu: gateup_bf16 is not 16-byte aligned");
    if (!aligned(h_bf16, 16)) return fail(FQ_ERR_ALIGN, "fq_geglu: h_bf16 is not 16-byte aligned");
    const fq::DeviceInfo* dev = nullptr;
    FQ_TRY(prepare(fn, &dev));
    return device_status(fn, fq::launch_geglu(static_cast<const uint16_t*>(gateup_bf16), M, F, ld_in,
                                              static_cast<uint16_t*>(h_bf16), ld_out,
                                              static_cast<hipStream_t>(stream)));
}

fq_status fq_linear_noalloc(const void* x_bf16, int32_t M, int32_t K, int64_t ldx, const float* gamma_folded,
                            float eps, const float* ascale, int32_t fold_after, int32_t hblock, int32_t abits,
                            const void* w_codes, const float* wscale, int32_t N, int32_t wbits, const float* bias,
                            const void* residual_bf16, int64_t ldr, void* y_bf16, int64_t ldy, void* stream) {
    return linear_impl("fq_linear_noalloc", x_bf16, M, K, ldx, gamma_folded, eps, ascale, fold_after, hblock, abits,
                       w_codes, wscale, N, wbits, bias, residual_bf16, ldr, y_bf16, ldy, 0, nullptr, 0, stream,
                       true);
}

size_t fq_linear_noalloc_max_bytes(void) { return fq::kNoallocScratchBytes; }

fq_status fq_linear_heads(const void* x_bf16, int32_t M, int32_t K, int64_t ldx, const float* gamma_folded,
                          float eps, const float* ascale, int32_t fold_after, int32_t hblock, int32_t abits,
                          const void* w_codes, const float* wscale, int32_t N, int32_t wbits, const float* bias,
                          const void* residual_bf16, int64_t ldr, int32_t head_dim, void* y_bf16, void* workspace,
                          size_t workspace_bytes, void* stream) {
    return linear_impl("fq_linear_heads", x_bf16, M, K, ldx, gamma_folded, eps, ascale, fold_after, hblock, abits,
                       w_codes, wscale, N, wbits, bias, residual_bf16, ldr, y_bf16, 0, head_dim, workspace,
                       workspace_bytes, stream);
}

}  // extern "C"
