// kda_api.cpp -- the C ABI (include/kda.h): host-side validation and launches.
//
// Every entry point validates all of its arguments before touching the HIP
// runtime, so a rejected call launches nothing and writes nothing. Messages
// for rejected calls are kept per thread and returned by kda_last_error().
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../../include/kda.h"
#include "kda_internal.h"

using namespace kda;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok()
{
    g_err.clear();
    return KDA_OK;
}

int hip_status(hipError_t e, const char* what)
{
    if (e == hipSuccess) return ok();
    return fail(KDA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool valid_dtype(kda_dtype d) { return d == KDA_F32 || d == KDA_BF16; }
size_t esize(kda_dtype d) { return d == KDA_F32 ? 4 : 2; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte range [p, p + n) of a tensor, for overlap checks.
struct Range {
    const char* p;
    size_t n;
};
Range rng(const void* p, size_t n) { return Range{static_cast<const char*>(p), n}; }
bool overlap(Range a, Range b)
{
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    return a.p < b.p + b.n && b.p < a.p + a.n;
}

#define REQUIRE(cond, code, ...)                \
    do {                                        \
        if (!(cond)) return fail(code, __VA_ARGS__); \
    } while (0)

// Log-retention floor of the chunked forms. Every factor 2^x those forms
// build spans the clamped log-retentions of at most one 16-token block, so
// |x| <= 16 |lower_bound| log2(e); at -5.4 that is 124.7, which keeps every
// factor a normal float32 (|x| < 126). NaN and positive floors (retention
// above one) are invalid; floors below -5.4 are not supported by the chunk
// form (the token-serial decode takes any floor <= 0).
constexpr float kChunkLowerBoundMin = -5.4f;

int check_lower_bound(const char* fn, float lb, bool chunked)
{
    REQUIRE(lb == lb && lb <= 0.0f, KDA_ERR_INVALID_ARG, "%s: lower_bound must be <= 0 and not NaN (got %g)", fn,
            (double)lb);
    if (chunked)
        REQUIRE(lb >= kChunkLowerBoundMin, KDA_ERR_UNSUPPORTED,
                "%s: lower_bound below %g is not supported by the chunk form (got %g)", fn,
                (double)kChunkLowerBoundMin, (double)lb);
    return KDA_OK;
}

// cu_seqlens on the host: cu[0] = 0, non-decreasing, cu[N] = T.
int check_cu(const int32_t* cu_dev, const int32_t* cu_host, int num_seqs, int64_t T, int64_t* seq_len)
{
    REQUIRE(num_seqs >= 1, KDA_ERR_INVALID_ARG, "num_seqs must be >= 1 (got %d)", num_seqs);
    REQUIRE((cu_dev == nullptr) == (cu_host == nullptr), KDA_ERR_INVALID_ARG,
            "cu_seqlens_dev and cu_seqlens_host must both be given or both be NULL");
    *seq_len = 0;
    if (!cu_host) {
        REQUIRE(T % num_seqs == 0, KDA_ERR_INVALID_ARG,
                "without cu_seqlens, num_tokens (%lld) must be a multiple of num_seqs (%d)",
                (long long)T, num_seqs);
        *seq_len = T / num_seqs;
        return KDA_OK;
    }
    REQUIRE(aligned16(cu_dev), KDA_ERR_INVALID_ARG, "cu_seqlens_dev must be 16-byte aligned");
    REQUIRE(cu_host[0] == 0, KDA_ERR_INVALID_ARG, "cu_seqlens[0] must be 0 (got %d)", cu_host[0]);
    for (int n = 0; n < num_seqs; ++n)
        REQUIRE(cu_host[n + 1] >= cu_host[n], KDA_ERR_INVALID_ARG,
                "cu_seqlens must be non-decreasing (cu[%d]=%d > cu[%d]=%d)", n, cu_host[n], n + 1,
                cu_host[n + 1]);
    REQUIRE((int64_t)cu_host[num_seqs] == T, KDA_ERR_INVALID_ARG,
            "cu_seqlens[num_seqs] (%d) must equal num_tokens (%lld)", cu_host[num_seqs], (long long)T);
    return KDA_OK;
}

}  // namespace

extern "C" {

const char* kda_last_error(void) { return g_err.c_str(); }

int kda_version(void) { return KDA_VERSION; }

size_t kda_state_bytes(int H, int dk, int dv, kda_dtype dtype)
{
    if (H <= 0 || dk <= 0 || dv <= 0 || !valid_dtype(dtype)) return 0;
    return (size_t)H * dk * dv * esize(dtype);
}

size_t kda_conv_state_bytes(int streams, int W, int C, kda_dtype dtype)
{
    if (streams <= 0 || W <= 1 || C <= 0 || !valid_dtype(dtype)) return 0;
    return (size_t)streams * (W - 1) * C * esize(dtype);
}

// ---------------------------------------------------------------- decode
static int decode_impl(const char* fn, const void* q, const void* k, const void* v, const void* g, const void* beta,
                       kda_dtype in_dtype, int B, int Tq, int H, int dk, int dv, float scale, float lower_bound,
                       void* state, void* token_states, kda_dtype state_dtype, void* o, kda_dtype out_dtype,
                       void* hip_stream)
{
    REQUIRE(q && k && v && g && beta && state && o, KDA_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
    REQUIRE(valid_dtype(in_dtype) && valid_dtype(out_dtype) && valid_dtype(state_dtype), KDA_ERR_INVALID_ARG,
            "%s: bad dtype", fn);
    REQUIRE(B >= 1 && H >= 1 && Tq >= 1, KDA_ERR_INVALID_ARG, "%s: B, H and the token count must be >= 1", fn);
    REQUIRE(dk == 128 && dv == 128, KDA_ERR_UNSUPPORTED, "%s: only dk = dv = 128 is supported (got %d, %d)", fn, dk,
            dv);
    REQUIRE((int64_t)B * H <= 0x7fffffff && (int64_t)B * Tq * H <= ((int64_t)1 << 40), KDA_ERR_INVALID_ARG,
            "%s: B*H too large", fn);
    if (int rc = check_lower_bound(fn, lower_bound, false); rc != KDA_OK) return rc;
    for (const void* p : {q, k, v, g, beta, (const void*)state, (const void*)token_states, (const void*)o})
        REQUIRE(!p || aligned16(p), KDA_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
    const size_t rows = (size_t)B * H, trows = rows * Tq, ss = 128 * 128 * esize(state_dtype);
    const Range rs = rng(state, rows * ss), ro = rng(o, trows * 128 * esize(out_dtype));
    const Range rt = rng(token_states, token_states ? trows * ss : 0);
    for (Range r : {rng(q, trows * 128 * esize(in_dtype)), rng(k, trows * 128 * esize(in_dtype)),
                    rng(v, trows * 128 * esize(in_dtype)), rng(g, trows * 128 * esize(in_dtype)),
                    rng(beta, trows * esize(in_dtype))}) {
        REQUIRE(!overlap(r, rs), KDA_ERR_INVALID_ARG, "%s: state overlaps an input", fn);
        REQUIRE(!overlap(r, ro), KDA_ERR_INVALID_ARG, "%s: o overlaps an input", fn);
        REQUIRE(!overlap(r, rt), KDA_ERR_INVALID_ARG, "%s: token_states overlaps an input", fn);
    }
    REQUIRE(!overlap(rs, ro), KDA_ERR_INVALID_ARG, "%s: o overlaps state", fn);
    REQUIRE(!overlap(rt, rs) && !overlap(rt, ro), KDA_ERR_INVALID_ARG, "%s: token_states overlaps state or o", fn);

    DecodeArgs a{q, k, v, g, beta, state, token_states, o, B, H, Tq, scale, lower_bound, (DType)in_dtype,
                 (DType)out_dtype, (DType)state_dtype};
    return hip_status(launch_decode(a, static_cast<hipStream_t>(hip_stream)), fn);
}

int kda_decode_step(const void* q, const void* k, const void* v, const void* g, const void* beta,
                    kda_dtype in_dtype, int B, int H, int dk, int dv, float scale,
                    float lower_bound, float* state, void* o, kda_dtype out_dtype,
                    void* hip_stream)
{
    return decode_impl("kda_decode_step", q, k, v, g, beta, in_dtype, B, 1, H, dk, dv, scale, lower_bound, state,
                       nullptr, KDA_F32, o, out_dtype, hip_stream);
}

int kda_decode_multi(const void* q, const void* k, const void* v, const void* g, const void* beta,
                     kda_dtype in_dtype, int B, int num_tokens, int H, int dk, int dv, float scale,
                     float lower_bound, void* state, void* token_states, kda_dtype state_dtype, void* o,
                     kda_dtype out_dtype, void* hip_stream)
{
    return decode_impl("kda_decode_multi", q, k, v, g, beta, in_dtype, B, num_tokens, H, dk, dv, scale, lower_bound,
                       state, token_states, state_dtype, o, out_dtype, hip_stream);
}

int kda_decode_commit(const void* token_states, const int32_t* accepted, int B, int num_tokens, int H, int dk,
                      int dv, void* state, kda_dtype state_dtype, void* hip_stream)
{
    REQUIRE(token_states && accepted && state, KDA_ERR_INVALID_ARG, "kda_decode_commit: null pointer");
    REQUIRE(valid_dtype(state_dtype), KDA_ERR_INVALID_ARG, "kda_decode_commit: bad dtype");
    REQUIRE(B >= 1 && H >= 1 && num_tokens >= 1, KDA_ERR_INVALID_ARG,
            "kda_decode_commit: B, H and the token count must be >= 1");
    REQUIRE(dk == 128 && dv == 128, KDA_ERR_UNSUPPORTED,
            "kda_decode_commit: only dk = dv = 128 is supported (got %d, %d)", dk, dv);
    REQUIRE((int64_t)B * H <= 0x7fffffff, KDA_ERR_INVALID_ARG, "kda_decode_commit: B*H too large");
    REQUIRE(aligned16(token_states) && aligned16(state), KDA_ERR_INVALID_ARG,
            "kda_decode_commit: token_states and state must be 16-byte aligned");
    const size_t rows = (size_t)B * H, ss = 128 * 128 * esize(state_dtype);
    const Range rs = rng(state, rows * ss);
    REQUIRE(!overlap(rs, rng(token_states, rows * num_tokens * ss)) && !overlap(rs, rng(accepted, (size_t)B * 4)),
            KDA_ERR_INVALID_ARG, "kda_decode_commit: state overlaps token_states or accepted");
    return hip_status(launch_decode_commit(token_states, accepted, state, B, num_tokens, H, (DType)state_dtype,
                                           static_cast<hipStream_t>(hip_stream)),
                      "kda_decode_commit");
}

int kda_state_convert(const void* src, kda_dtype src_dtype, void* dst, kda_dtype dst_dtype, int64_t count,
                      void* hip_stream)
{
    REQUIRE(count >= 0, KDA_ERR_INVALID_ARG, "kda_state_convert: negative count");
    REQUIRE(count == 0 || (src && dst), KDA_ERR_INVALID_ARG, "kda_state_convert: null pointer");
    REQUIRE(valid_dtype(src_dtype) && valid_dtype(dst_dtype), KDA_ERR_INVALID_ARG, "kda_state_convert: bad dtype");
    REQUIRE((!src || aligned16(src)) && (!dst || aligned16(dst)), KDA_ERR_INVALID_ARG,
            "kda_state_convert: pointers must be 16-byte aligned");
    REQUIRE(!overlap(rng(src, (size_t)count * esize(src_dtype)), rng(dst, (size_t)count * esize(dst_dtype))),
            KDA_ERR_INVALID_ARG, "kda_state_convert: src and dst overlap");
    return hip_status(launch_convert(src, (DType)src_dtype, dst, (DType)dst_dtype, count,
                                     static_cast<hipStream_t>(hip_stream)),
                      "kda_state_convert");
}

// ---------------------------------------------------------------- conv
int kda_conv_state_update(const void* x, int64_t x_ld, void* conv_state, const void* weight, const void* bias,
                          kda_dtype dtype, int B, int C, int W, int apply_silu,
                          int l2norm_group, float l2norm_eps, void* y, void* hip_stream)
{
    REQUIRE(x && conv_state && weight && y, KDA_ERR_INVALID_ARG, "kda_conv_state_update: null pointer");
    REQUIRE(valid_dtype(dtype), KDA_ERR_INVALID_ARG, "kda_conv_state_update: bad dtype");
    REQUIRE(B >= 1 && C >= 2, KDA_ERR_INVALID_ARG, "kda_conv_state_update: bad B or C");
    REQUIRE(W >= 2 && W <= 8, KDA_ERR_UNSUPPORTED, "kda_conv_state_update: W must be in [2, 8] (got %d)", W);
    REQUIRE(C % 128 == 0, KDA_ERR_UNSUPPORTED, "kda_conv_state_update: C must be a multiple of 128 (got %d)", C);
    REQUIRE(l2norm_group == 0 || l2norm_group == 128, KDA_ERR_UNSUPPORTED,
            "kda_conv_state_update: l2norm_group must be 0 or 128 (got %d)", l2norm_group);
    REQUIRE(x_ld >= C && x_ld % 8 == 0, KDA_ERR_INVALID_ARG,
            "kda_conv_state_update: x_ld must be >= C and a multiple of 8");
    for (const void* p : {x, (const void*)conv_state, weight, bias, (const void*)y})
        REQUIRE(!p || aligned16(p), KDA_ERR_INVALID_ARG, "kda_conv_state_update: pointers must be 16-byte aligned");
    const size_t es = esize(dtype);
    const Range ry = rng(y, (size_t)B * C * es), rs = rng(conv_state, (size_t)B * (W - 1) * C * es);
    const Range rx = rng(x, ((size_t)(B - 1) * x_ld + C) * es), rw = rng(weight, (size_t)C * W * es),
                rb = rng(bias, bias ? (size_t)C * es : 0);
    REQUIRE(!overlap(ry, rx) && !overlap(ry, rs) && !overlap(ry, rw) && !overlap(ry, rb),
            KDA_ERR_INVALID_ARG, "kda_conv_state_update: y overlaps another tensor");
    REQUIRE(!overlap(rs, rx) && !overlap(rs, rw) && !overlap(rs, rb), KDA_ERR_INVALID_ARG,
            "kda_conv_state_update: conv_state overlaps an input");

    ConvUpdateArgs a{x, x_ld, conv_state, weight, bias, y, B, C, W, apply_silu ? 1 : 0, l2norm_group,
                     l2norm_eps, (DType)dtype};
    return hip_status(launch_conv_update(a, static_cast<hipStream_t>(hip_stream)), "kda_conv_state_update");
}

int kda_conv_prefill(const void* x, int64_t x_ld, int64_t num_tokens, int C, int W,
                     const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs,
                     const void* weight, const void* bias, const void* conv_state_in,
                     void* conv_state_out, int apply_silu, int l2norm_group, float l2norm_eps,
                     void* y, int64_t y_ld, kda_dtype dtype, void* hip_stream)
{
    REQUIRE(x && weight && y, KDA_ERR_INVALID_ARG, "kda_conv_prefill: null pointer");
    REQUIRE(valid_dtype(dtype), KDA_ERR_INVALID_ARG, "kda_conv_prefill: bad dtype");
    REQUIRE(num_tokens >= 0 && C >= 2, KDA_ERR_INVALID_ARG, "kda_conv_prefill: bad num_tokens or C");
    REQUIRE(W >= 2 && W <= 8, KDA_ERR_UNSUPPORTED, "kda_conv_prefill: W must be in [2, 8] (got %d)", W);
    REQUIRE(C % 128 == 0, KDA_ERR_UNSUPPORTED, "kda_conv_prefill: C must be a multiple of 128 (got %d)", C);
    REQUIRE(l2norm_group == 0 || l2norm_group == 128, KDA_ERR_UNSUPPORTED,
            "kda_conv_prefill: l2norm_group must be 0 or 128 (got %d)", l2norm_group);
    REQUIRE(x_ld >= C && y_ld >= C && x_ld % 8 == 0 && y_ld % 8 == 0, KDA_ERR_INVALID_ARG,
            "kda_conv_prefill: x_ld and y_ld must be >= C and multiples of 8");
    for (const void* p : {x, weight, bias, conv_state_in, (const void*)conv_state_out, (const void*)y})
        REQUIRE(!p || aligned16(p), KDA_ERR_INVALID_ARG, "kda_conv_prefill: pointers must be 16-byte aligned");
    int64_t seq_len = 0;
    int rc = check_cu(cu_seqlens_dev, cu_seqlens_host, num_seqs, num_tokens, &seq_len);
    if (rc != KDA_OK) return rc;
    const size_t es = esize(dtype);
    const size_t rows_bytes_y = num_tokens > 0 ? ((size_t)(num_tokens - 1) * y_ld + C) * es : 0;
    const size_t rows_bytes_x = num_tokens > 0 ? ((size_t)(num_tokens - 1) * x_ld + C) * es : 0;
    const size_t sbytes = (size_t)num_seqs * (W - 1) * C * es;
    const Range ry = rng(y, rows_bytes_y), rx = rng(x, rows_bytes_x), rso = rng(conv_state_out, conv_state_out ? sbytes : 0),
                rsi = rng(conv_state_in, conv_state_in ? sbytes : 0);
    REQUIRE(!overlap(ry, rx) && !overlap(ry, rsi) && !overlap(ry, rso), KDA_ERR_INVALID_ARG,
            "kda_conv_prefill: y overlaps an input or the output state");
    REQUIRE(!overlap(rso, rx) && !overlap(rso, rsi), KDA_ERR_INVALID_ARG,
            "kda_conv_prefill: conv_state_out overlaps x or conv_state_in");

    ConvPrefillArgs a{};
    a.x = x; a.x_ld = x_ld; a.y_ld = y_ld; a.num_tokens = num_tokens; a.C = C; a.W = W;
    a.num_seqs = num_seqs; a.apply_silu = apply_silu ? 1 : 0; a.l2_group = l2norm_group;
    a.seq_len = seq_len; a.cu_seqlens = cu_seqlens_dev; a.weight = weight; a.bias = bias;
    a.state_in = conv_state_in; a.state_out = conv_state_out; a.y = y; a.l2_eps = l2norm_eps;
    a.dtype = (DType)dtype;
    return hip_status(launch_conv_prefill(a, static_cast<hipStream_t>(hip_stream)), "kda_conv_prefill");
}

// ---------------------------------------------------------------- gate / epilogue
int kda_gate_prologue(const void* f, int64_t f_ld, const void* b, int64_t b_ld,
                      const float* A_log, int64_t num_tokens, int H, int dk, float lower_bound,
                      kda_dtype in_dtype, void* g_out, void* beta_out, kda_dtype out_dtype,
                      void* hip_stream)
{
    REQUIRE(f && b && A_log && g_out && beta_out, KDA_ERR_INVALID_ARG, "kda_gate_prologue: null pointer");
    REQUIRE(valid_dtype(in_dtype) && valid_dtype(out_dtype), KDA_ERR_INVALID_ARG, "kda_gate_prologue: bad dtype");
    REQUIRE(num_tokens >= 0 && H >= 1, KDA_ERR_INVALID_ARG, "kda_gate_prologue: bad sizes");
    REQUIRE(dk == 128, KDA_ERR_UNSUPPORTED, "kda_gate_prologue: only dk = 128 is supported");
    if (int rc = check_lower_bound("kda_gate_prologue", lower_bound, false); rc != KDA_OK) return rc;
    REQUIRE(f_ld >= (int64_t)H * dk && f_ld % 8 == 0 && b_ld >= H, KDA_ERR_INVALID_ARG,
            "kda_gate_prologue: f_ld must be >= H*dk and a multiple of 8; b_ld >= H");
    for (const void* p : {f, b, (const void*)A_log, (const void*)g_out, (const void*)beta_out})
        REQUIRE(aligned16(p), KDA_ERR_INVALID_ARG, "kda_gate_prologue: pointers must be 16-byte aligned");
    const size_t ei = esize(in_dtype), eo = esize(out_dtype);
    const Range rg = rng(g_out, (size_t)num_tokens * H * dk * eo), rb = rng(beta_out, (size_t)num_tokens * H * eo);
    const Range rf = rng(f, num_tokens ? ((size_t)(num_tokens - 1) * f_ld + (size_t)H * dk) * ei : 0);
    const Range rbi = rng(b, num_tokens ? ((size_t)(num_tokens - 1) * b_ld + H) * ei : 0);
    REQUIRE(!overlap(rg, rf) && !overlap(rg, rbi) && !overlap(rb, rf) && !overlap(rb, rbi) && !overlap(rg, rb),
            KDA_ERR_INVALID_ARG, "kda_gate_prologue: outputs overlap inputs or each other");
    GateArgs a{f, b, f_ld, b_ld, num_tokens, A_log, g_out, beta_out, H, dk, lower_bound,
               (DType)in_dtype, (DType)out_dtype};
    return hip_status(launch_gate(a, static_cast<hipStream_t>(hip_stream)), "kda_gate_prologue");
}

int kda_output_norm_gate(const void* o, kda_dtype o_dtype, const void* gate, int64_t gate_ld,
                         const float* norm_weight, int64_t num_tokens, int H, int dv, float eps,
                         void* y, kda_dtype y_dtype, void* hip_stream)
{
    REQUIRE(o && gate && norm_weight && y, KDA_ERR_INVALID_ARG, "kda_output_norm_gate: null pointer");
    REQUIRE(valid_dtype(o_dtype) && valid_dtype(y_dtype), KDA_ERR_INVALID_ARG, "kda_output_norm_gate: bad dtype");
    REQUIRE(num_tokens >= 0 && H >= 1, KDA_ERR_INVALID_ARG, "kda_output_norm_gate: bad sizes");
    REQUIRE(dv == 128, KDA_ERR_UNSUPPORTED, "kda_output_norm_gate: only dv = 128 is supported");
    REQUIRE(gate_ld >= (int64_t)H * dv && gate_ld % 8 == 0, KDA_ERR_INVALID_ARG,
            "kda_output_norm_gate: gate_ld must be >= H*dv and a multiple of 8");
    for (const void* p : {o, gate, (const void*)norm_weight, (const void*)y})
        REQUIRE(aligned16(p), KDA_ERR_INVALID_ARG, "kda_output_norm_gate: pointers must be 16-byte aligned");
    const Range ry = rng(y, (size_t)num_tokens * H * dv * esize(y_dtype));
    const Range ro = rng(o, (size_t)num_tokens * H * dv * esize(o_dtype));
    const Range rgt = rng(gate, num_tokens ? ((size_t)(num_tokens - 1) * gate_ld + (size_t)H * dv) * esize(y_dtype) : 0);
    REQUIRE(!overlap(ry, ro) && !overlap(ry, rgt), KDA_ERR_INVALID_ARG, "kda_output_norm_gate: y overlaps an input");
    NormGateArgs a{o, gate, gate_ld, num_tokens, norm_weight, y, H, dv, eps, (DType)o_dtype, (DType)y_dtype};
    return hip_status(launch_norm_gate(a, static_cast<hipStream_t>(hip_stream)), "kda_output_norm_gate");
}

// ---------------------------------------------------------------- block FP8
int kda_gemv_fp8(const void* x, int64_t ldx, const uint8_t* w, int64_t ldw, const float* w_scale, int64_t ws_ld,
                 void* y, int64_t ldy, int M, int64_t N, int64_t K, kda_dtype x_dtype, kda_dtype y_dtype,
                 void* hip_stream)
{
    REQUIRE(x && w && w_scale && y, KDA_ERR_INVALID_ARG, "kda_gemv_fp8: null pointer");
    REQUIRE(valid_dtype(x_dtype) && valid_dtype(y_dtype), KDA_ERR_INVALID_ARG, "kda_gemv_fp8: bad dtype");
    REQUIRE(x_dtype == KDA_BF16, KDA_ERR_UNSUPPORTED, "kda_gemv_fp8: x must be bfloat16");
    REQUIRE(M >= 1 && M <= 8, KDA_ERR_UNSUPPORTED, "kda_gemv_fp8: 1 <= M <= 8 rows (got %d)", M);
    REQUIRE(N >= 1 && K >= 128, KDA_ERR_INVALID_ARG, "kda_gemv_fp8: bad sizes");
    REQUIRE(K % 128 == 0, KDA_ERR_UNSUPPORTED, "kda_gemv_fp8: K must be a multiple of 128 (the scale block)");
    REQUIRE(ldx >= K && ldx % 8 == 0 && ldw >= K && ldw % 16 == 0 && ws_ld >= K / 128 && ldy >= N,
            KDA_ERR_INVALID_ARG,
            "kda_gemv_fp8: ldx >= K (multiple of 8), ldw >= K (multiple of 16), ws_ld >= K/128, ldy >= N");
    REQUIRE(aligned16(x) && aligned16(w) && aligned16(y) && ((uintptr_t)w_scale % 4 == 0), KDA_ERR_INVALID_ARG,
            "kda_gemv_fp8: x, w and y must be 16-byte aligned");
    const Range ry = rng(y, ((size_t)(M - 1) * ldy + N) * esize(y_dtype));
    REQUIRE(!overlap(ry, rng(x, ((size_t)(M - 1) * ldx + K) * 2)) && !overlap(ry, rng(w, (size_t)(N - 1) * ldw + K)) &&
                !overlap(ry, rng(w_scale, ((size_t)((N + 127) / 128 - 1) * ws_ld + K / 128) * 4)),
            KDA_ERR_INVALID_ARG, "kda_gemv_fp8: y overlaps an input");
    Fp8GemvArgs a{x, w, w_scale, y, ldx, ldw, ws_ld, ldy, N, K, M, (DType)y_dtype};
    return hip_status(launch_gemv_fp8(a, static_cast<hipStream_t>(hip_stream)), "kda_gemv_fp8");
}

int kda_quantize_fp8(const void* x, int64_t ldx, kda_dtype x_dtype, int64_t M, int64_t K, uint8_t* codes,
                     int64_t ldc, float* scales, int64_t ld_scale, void* hip_stream)
{
    REQUIRE(x && codes && scales, KDA_ERR_INVALID_ARG, "kda_quantize_fp8: null pointer");
    REQUIRE(valid_dtype(x_dtype), KDA_ERR_INVALID_ARG, "kda_quantize_fp8: bad dtype");
    REQUIRE(M >= 0 && K >= 128, KDA_ERR_INVALID_ARG, "kda_quantize_fp8: bad sizes");
    REQUIRE(K % 128 == 0, KDA_ERR_UNSUPPORTED, "kda_quantize_fp8: K must be a multiple of 128 (the group)");
    REQUIRE(ldx >= K && ldx % 8 == 0 && ldc >= K && ldc % 8 == 0 && ld_scale >= K / 128, KDA_ERR_INVALID_ARG,
            "kda_quantize_fp8: ldx >= K and ldc >= K (multiples of 8), ld_scale >= K/128");
    REQUIRE(aligned16(x) && ((uintptr_t)codes % 8 == 0) && ((uintptr_t)scales % 4 == 0), KDA_ERR_INVALID_ARG,
            "kda_quantize_fp8: x must be 16-byte aligned, codes 8-byte aligned");
    if (M == 0) return KDA_OK;
    const Range rx = rng(x, ((size_t)(M - 1) * ldx + K) * esize(x_dtype));
    const Range rc = rng(codes, (size_t)(M - 1) * ldc + K), rs = rng(scales, ((size_t)(M - 1) * ld_scale + K / 128) * 4);
    REQUIRE(!overlap(rc, rx) && !overlap(rs, rx) && !overlap(rc, rs), KDA_ERR_INVALID_ARG,
            "kda_quantize_fp8: outputs overlap each other or the input");
    QuantFp8Args a{x, codes, scales, ldx, ldc, ld_scale, M, K, (DType)x_dtype};
    return hip_status(launch_quantize_fp8(a, static_cast<hipStream_t>(hip_stream)), "kda_quantize_fp8");
}

int kda_gemm_fp8(const uint8_t* x, int64_t ldx, const float* x_scale, int64_t xs_ld, const uint8_t* w, int64_t ldw,
                 const float* w_scale, int64_t ws_ld, void* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                 kda_dtype y_dtype, void* hip_stream)
{
    REQUIRE(x && x_scale && w && w_scale && y, KDA_ERR_INVALID_ARG, "kda_gemm_fp8: null pointer");
    REQUIRE(valid_dtype(y_dtype), KDA_ERR_INVALID_ARG, "kda_gemm_fp8: bad dtype");
    REQUIRE(M >= 0 && N >= 1 && K >= 128, KDA_ERR_INVALID_ARG, "kda_gemm_fp8: bad sizes");
    REQUIRE(K % 128 == 0, KDA_ERR_UNSUPPORTED, "kda_gemm_fp8: K must be a multiple of 128 (the scale block)");
    REQUIRE(ldx >= K && ldx % 16 == 0 && ldw >= K && ldw % 16 == 0 && xs_ld >= K / 128 && ws_ld >= K / 128 &&
                ldy >= N,
            KDA_ERR_INVALID_ARG,
            "kda_gemm_fp8: ldx, ldw >= K (multiples of 16), xs_ld, ws_ld >= K/128, ldy >= N");
    REQUIRE(aligned16(x) && aligned16(w) && ((uintptr_t)x_scale % 4 == 0) && ((uintptr_t)w_scale % 4 == 0) &&
                ((uintptr_t)y % esize(y_dtype) == 0),
            KDA_ERR_INVALID_ARG, "kda_gemm_fp8: x and w must be 16-byte aligned");
    // the matrix-core kernel addresses a tile's rows through 32-bit offsets
    REQUIRE(256 * std::max(ldx, ldw) + K < ((int64_t)1 << 31), KDA_ERR_UNSUPPORTED,
            "kda_gemm_fp8: row strides too large");
    if (M == 0) return KDA_OK;
    const Range ry = rng(y, ((size_t)(M - 1) * ldy + N) * esize(y_dtype));
    for (Range r : {rng(x, (size_t)(M - 1) * ldx + K), rng(w, (size_t)(N - 1) * ldw + K),
                    rng(x_scale, ((size_t)(M - 1) * xs_ld + K / 128) * 4),
                    rng(w_scale, ((size_t)((N + 127) / 128 - 1) * ws_ld + K / 128) * 4)})
        REQUIRE(!overlap(ry, r), KDA_ERR_INVALID_ARG, "kda_gemm_fp8: y overlaps an input");
    Fp8GemvArgs a{x, w, w_scale, y, ldx, ldw, ws_ld, ldy, N, K, M, (DType)y_dtype, x_scale, xs_ld};
    const hipStream_t st = static_cast<hipStream_t>(hip_stream);
    // a few rows (decode): the weight-streaming forms of kda_gemv_fp8;
    // more: the matrix-core GEMM
    return hip_status(M <= 8 ? launch_gemv_fp8(a, st) : launch_gemm_fp8(a, st), "kda_gemm_fp8");
}

int kda_output_norm_gate_fp8(const void* o, kda_dtype o_dtype, const void* gate, int64_t gate_ld,
                             kda_dtype gate_dtype, const float* norm_weight, int64_t num_tokens, int H, int dv,
                             float eps, uint8_t* y_codes, float* y_scales, void* hip_stream)
{
    REQUIRE(o && gate && norm_weight && y_codes && y_scales, KDA_ERR_INVALID_ARG,
            "kda_output_norm_gate_fp8: null pointer");
    REQUIRE(valid_dtype(o_dtype) && valid_dtype(gate_dtype), KDA_ERR_INVALID_ARG,
            "kda_output_norm_gate_fp8: bad dtype");
    REQUIRE(num_tokens >= 0 && H >= 1, KDA_ERR_INVALID_ARG, "kda_output_norm_gate_fp8: bad sizes");
    REQUIRE(dv == 128, KDA_ERR_UNSUPPORTED, "kda_output_norm_gate_fp8: only dv = 128 is supported");
    REQUIRE(gate_ld >= (int64_t)H * dv && gate_ld % 8 == 0, KDA_ERR_INVALID_ARG,
            "kda_output_norm_gate_fp8: gate_ld must be >= H*dv and a multiple of 8");
    for (const void* p : {o, gate, (const void*)norm_weight, (const void*)y_codes, (const void*)y_scales})
        REQUIRE(aligned16(p), KDA_ERR_INVALID_ARG, "kda_output_norm_gate_fp8: pointers must be 16-byte aligned");
    const size_t rows = (size_t)num_tokens * H;
    const Range rc = rng(y_codes, rows * dv), rsc = rng(y_scales, rows * 4);
    const Range ro = rng(o, rows * dv * esize(o_dtype));
    const Range rgt = rng(gate, num_tokens ? ((size_t)(num_tokens - 1) * gate_ld + (size_t)H * dv) * esize(gate_dtype) : 0);
    for (Range r : {ro, rgt, rng(norm_weight, (size_t)dv * 4)})
        REQUIRE(!overlap(rc, r) && !overlap(rsc, r), KDA_ERR_INVALID_ARG,
                "kda_output_norm_gate_fp8: an output overlaps an input");
    REQUIRE(!overlap(rc, rsc), KDA_ERR_INVALID_ARG, "kda_output_norm_gate_fp8: y_codes overlaps y_scales");
    NormGateFp8Args a{o, gate, gate_ld, num_tokens, norm_weight, y_codes, y_scales, H, eps, (DType)o_dtype,
                      (DType)gate_dtype};
    return hip_status(launch_norm_gate_fp8(a, static_cast<hipStream_t>(hip_stream)), "kda_output_norm_gate_fp8");
}

// ---------------------------------------------------------------- prefill
namespace {
constexpr int64_t kChunk = 64;          // chunk of the bfloat16 forms
constexpr int64_t kWindowChunks = 32;   // recommended window of the two-pass form (measured best of 16..48)
size_t state_carry_bytes(int64_t units) { return (size_t)units * 128 * 128 * sizeof(float); }
}  // namespace

size_t kda_prefill_workspace_bytes(int64_t num_tokens, int num_seqs, int H, int dk, int dv,
                                   kda_dtype in_dtype)
{
    if (in_dtype != KDA_BF16 || num_tokens <= 0 || num_seqs < 1 || H < 1 || dk != 128 || dv != 128) return 0;
    const int64_t units = (int64_t)num_seqs * H;
    const int64_t max_chunks = (num_tokens + kChunk - 1) / kChunk;  // bounds every sequence's chunk count
    const int64_t nwin = std::min(max_chunks, kWindowChunks);
    size_t bytes = (size_t)(units * nwin) * prefill_split_slot_bytes();
    if (nwin < max_chunks) bytes += state_carry_bytes(units);
    return bytes;
}

// the gate inputs of kda_prefill_gated
struct GateIn {
    const void* f;
    int64_t f_ld;
    const void* b;
    int64_t b_ld;
    const float* A_log;
};

static int prefill_impl(const void* q, const void* k, const void* v, const void* g, const void* beta,
                        kda_dtype in_dtype, int64_t num_tokens, int H, int dk, int dv,
                        const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs,
                        float scale, float lower_bound, const float* initial_state, float* final_state,
                        void* o, kda_dtype out_dtype, void* workspace, size_t workspace_bytes,
                        int64_t snap_interval, int64_t snap_slots, float* snapshots, void* hip_stream,
                        bool static_ws = false, const GateIn* gate = nullptr)
{
    const char* fn = gate ? "kda_prefill_gated" : "kda_prefill";
    if (gate) {
        REQUIRE(in_dtype == KDA_BF16, KDA_ERR_UNSUPPORTED, "%s: bfloat16 inputs only", fn);
        REQUIRE(workspace != nullptr, KDA_ERR_WORKSPACE, "%s: a workspace is required (two-pass form)", fn);
        REQUIRE(num_tokens == 0 || (gate->f && gate->b && gate->A_log), KDA_ERR_INVALID_ARG,
                "%s: null f, b or A_log", fn);
        REQUIRE(gate->f_ld >= (int64_t)H * 128 && gate->f_ld % 8 == 0 && gate->f_ld < ((int64_t)1 << 24),
                KDA_ERR_INVALID_ARG, "%s: f_ld must be a multiple of 8 in [H*128, 2^24) (got %lld)", fn,
                (long long)gate->f_ld);
        REQUIRE(gate->b_ld >= H && gate->b_ld < ((int64_t)1 << 24), KDA_ERR_INVALID_ARG,
                "%s: b_ld must lie in [H, 2^24) (got %lld)", fn, (long long)gate->b_ld);
        REQUIRE(aligned16(gate->f) && ((uintptr_t)gate->b & 1) == 0, KDA_ERR_INVALID_ARG,
                "%s: f must be 16-byte and b 2-byte aligned", fn);
        g = gate->f;  // stand-ins for the pointer checks below; never read as g or beta
        beta = gate->b;
    }
    REQUIRE(valid_dtype(in_dtype) && valid_dtype(out_dtype), KDA_ERR_INVALID_ARG, "kda_prefill: bad dtype");
    REQUIRE(num_tokens >= 0 && H >= 1, KDA_ERR_INVALID_ARG, "kda_prefill: bad num_tokens or H");
    REQUIRE(dk == 128 && dv == 128, KDA_ERR_UNSUPPORTED,
            "kda_prefill: only dk = dv = 128 is supported (got %d, %d)", dk, dv);
    if (int rc = check_lower_bound("kda_prefill", lower_bound, true); rc != KDA_OK) return rc;
    REQUIRE(num_tokens == 0 || (q && k && v && g && beta && o), KDA_ERR_INVALID_ARG,
            "kda_prefill: null tensor pointer");
    for (const void* p : {q, k, v, g, gate ? nullptr : beta, (const void*)initial_state, (const void*)final_state,
                          (const void*)o, (const void*)workspace, (const void*)snapshots})
        REQUIRE(!p || aligned16(p), KDA_ERR_INVALID_ARG, "kda_prefill: pointers must be 16-byte aligned");
    int64_t seq_len = 0;
    int rc = check_cu(cu_seqlens_dev, cu_seqlens_host, num_seqs, num_tokens, &seq_len);
    if (rc != KDA_OK) return rc;
    REQUIRE((int64_t)num_seqs * H * 2 <= 0x7fffffff, KDA_ERR_INVALID_ARG, "kda_prefill: num_seqs*H too large");

    // the two-pass form runs for bfloat16 inputs when a workspace is given
    // (kda_prefill_noalloc: always, in the static scratch)
    const bool split = in_dtype == KDA_BF16 && (workspace != nullptr || static_ws);
    const int64_t units = (int64_t)num_seqs * H;
    int64_t max_len = seq_len;
    if (cu_seqlens_host)
        for (int n = 0; n < num_seqs; ++n)
            max_len = std::max<int64_t>(max_len, (int64_t)cu_seqlens_host[n + 1] - cu_seqlens_host[n]);
    const int64_t max_chunks = (max_len + kChunk - 1) / kChunk;
    if (snapshots) {
        REQUIRE(snap_interval >= kChunk && snap_interval % kChunk == 0, KDA_ERR_INVALID_ARG,
                "kda_prefill_snapshots: snapshot_interval must be a positive multiple of %lld (got %lld)",
                (long long)kChunk, (long long)snap_interval);
        REQUIRE(snap_slots >= max_len / snap_interval, KDA_ERR_INVALID_ARG,
                "kda_prefill_snapshots: %lld snapshot slots per sequence needed (got %lld)",
                (long long)(max_len / snap_interval), (long long)snap_slots);
    }
    if (split) {
        const size_t slot = prefill_split_slot_bytes();
        const size_t whole = (size_t)(units * std::max<int64_t>(max_chunks, 1)) * slot;
        const size_t least = (size_t)units * slot + state_carry_bytes(units);
        if (static_ws) {
            REQUIRE(std::min(whole, least) <= kStaticScratchBytes, KDA_ERR_WORKSPACE,
                    "kda_prefill_noalloc: %lld (sequence, head) units need at least %zu bytes of workspace, more "
                    "than the %zu-byte static scratch (at most %zu units)",
                    (long long)units, std::min(whole, least), kStaticScratchBytes,
                    kStaticScratchBytes / (slot + (size_t)128 * 128 * sizeof(float)));
        } else {
            REQUIRE(workspace_bytes >= std::min(whole, least), KDA_ERR_WORKSPACE,
                    "kda_prefill: workspace of at least %zu bytes required (got %zu)", std::min(whole, least),
                    workspace_bytes);
        }
    }

    if (static_ws && split) {
        // every argument is valid: look up this device's scratch array
        void* p = nullptr;
        const hipError_t e = prefill_static_scratch(&p);
        if (e != hipSuccess) return hip_status(e, "kda_prefill_noalloc: static scratch");
        workspace = p;
        workspace_bytes = kStaticScratchBytes;
    }
    const size_t ei = esize(in_dtype), T = (size_t)num_tokens;
    const size_t sbytes = (size_t)num_seqs * H * 128 * 128 * 4;
    const Range ro = rng(o, T * H * 128 * esize(out_dtype));
    const Range rs0 = rng(initial_state, initial_state ? sbytes : 0), rsT = rng(final_state, final_state ? sbytes : 0);
    const Range rws = rng(workspace, split ? workspace_bytes : 0);
    const Range rsn = rng(snapshots, snapshots ? (size_t)num_seqs * snap_slots * H * 128 * 128 * 4 : 0);
    const Range rg = gate ? rng(g, T ? ((T - 1) * (size_t)gate->f_ld + H * 128) * ei : 0) : rng(g, T * H * 128 * ei);
    const Range rb = gate ? rng(beta, T ? ((T - 1) * (size_t)gate->b_ld + H) * ei : 0) : rng(beta, T * H * ei);
    for (const Range& r : {rng(q, T * H * 128 * ei), rng(k, T * H * 128 * ei), rng(v, T * H * 128 * ei),
                           rg, rb, rs0, ro, rsT, rws})
        REQUIRE(!overlap(r, rsn), KDA_ERR_INVALID_ARG, "kda_prefill_snapshots: snapshots overlap another tensor");
    const Range ins[] = {rng(q, T * H * 128 * ei), rng(k, T * H * 128 * ei), rng(v, T * H * 128 * ei),
                         rg, rb, rs0};
    for (const Range& r : ins) {
        REQUIRE(!overlap(r, ro), KDA_ERR_INVALID_ARG, "kda_prefill: o overlaps an input");
        if (r.p != rs0.p) REQUIRE(!overlap(r, rsT), KDA_ERR_INVALID_ARG, "kda_prefill: final_state overlaps an input");
        REQUIRE(!overlap(r, rws), KDA_ERR_INVALID_ARG, "kda_prefill: workspace overlaps an input");
    }
    REQUIRE(!overlap(ro, rsT), KDA_ERR_INVALID_ARG, "kda_prefill: o overlaps final_state");
    REQUIRE(!overlap(rws, ro) && !overlap(rws, rsT), KDA_ERR_INVALID_ARG,
            "kda_prefill: workspace overlaps o or final_state");
    REQUIRE(!overlap(rs0, rsT) || (initial_state == final_state), KDA_ERR_INVALID_ARG,
            "kda_prefill: initial_state and final_state overlap without being the same buffer");

    PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.cu_seqlens = cu_seqlens_dev; a.seq_len = seq_len;
    a.s0 = initial_state; a.sT = final_state; a.o = o;
    a.num_seqs = num_seqs; a.H = H; a.scale = scale; a.lower_bound = lower_bound;
    a.in_dtype = (DType)in_dtype; a.out_dtype = (DType)out_dtype;
    a.snap = snapshots; a.snap_interval = snapshots ? snap_interval : 0; a.snap_slots = snapshots ? snap_slots : 0;
    if (gate) {
        a.g = a.beta = nullptr;
        a.gate_f = gate->f; a.gate_f_ld = gate->f_ld;
        a.gate_b = gate->b; a.gate_b_ld = gate->b_ld;
        a.A_log = gate->A_log;
    }
    const hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (split)
        return hip_status(launch_prefill_split(a, workspace, workspace_bytes, max_chunks, cu_seqlens_host, st), "kda_prefill");
    return hip_status(launch_prefill(a, st), "kda_prefill");
}

int kda_prefill(const void* q, const void* k, const void* v, const void* g, const void* beta,
                kda_dtype in_dtype, int64_t num_tokens, int H, int dk, int dv,
                const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs,
                float scale, float lower_bound, const float* initial_state, float* final_state,
                void* o, kda_dtype out_dtype, void* workspace, size_t workspace_bytes,
                void* hip_stream)
{
    return prefill_impl(q, k, v, g, beta, in_dtype, num_tokens, H, dk, dv, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                        scale, lower_bound, initial_state, final_state, o, out_dtype, workspace, workspace_bytes, 0, 0,
                        nullptr, hip_stream);
}

int kda_prefill_snapshots(const void* q, const void* k, const void* v, const void* g, const void* beta,
                          kda_dtype in_dtype, int64_t num_tokens, int H, int dk, int dv,
                          const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs,
                          float scale, float lower_bound, const float* initial_state, float* final_state,
                          void* o, kda_dtype out_dtype, void* workspace, size_t workspace_bytes,
                          int64_t snapshot_interval, int64_t snapshot_slots, float* snapshots, void* hip_stream)
{
    REQUIRE(snapshots, KDA_ERR_INVALID_ARG, "kda_prefill_snapshots: null snapshots");
    return prefill_impl(q, k, v, g, beta, in_dtype, num_tokens, H, dk, dv, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                        scale, lower_bound, initial_state, final_state, o, out_dtype, workspace, workspace_bytes,
                        snapshot_interval, snapshot_slots, snapshots, hip_stream);
}

int kda_prefill_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta,
                        kda_dtype in_dtype, int64_t num_tokens, int H, int dk, int dv,
                        const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs,
                        float scale, float lower_bound, const float* initial_state, float* final_state,
                        void* o, kda_dtype out_dtype, void* hip_stream)
{
    return prefill_impl(q, k, v, g, beta, in_dtype, num_tokens, H, dk, dv, cu_seqlens_dev, cu_seqlens_host, num_seqs,
                        scale, lower_bound, initial_state, final_state, o, out_dtype, nullptr, 0, 0, 0, nullptr,
                        hip_stream, true);
}

size_t kda_prefill_noalloc_scratch_bytes(void) { return kStaticScratchBytes; }

int kda_prefill_gated(const void* q, const void* k, const void* v, const void* f, int64_t f_ld, const void* b,
                      int64_t b_ld, const float* A_log, kda_dtype in_dtype, int64_t num_tokens, int H, int dk, int dv,
                      const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs,
                      float scale, float lower_bound, const float* initial_state, float* final_state,
                      void* o, kda_dtype out_dtype, void* workspace, size_t workspace_bytes, void* hip_stream)
{
    const GateIn gate{f, f_ld, b, b_ld, A_log};
    return prefill_impl(q, k, v, nullptr, nullptr, in_dtype, num_tokens, H, dk, dv, cu_seqlens_dev, cu_seqlens_host,
                        num_seqs, scale, lower_bound, initial_state, final_state, o, out_dtype, workspace,
                        workspace_bytes, 0, 0, nullptr, hip_stream, false, &gate);
}

// ---------------------------------------------------------------- segment maps
int kda_prefill_segment_maps(const void* k, const void* v, const void* g, const void* beta, kda_dtype in_dtype,
                             int64_t num_tokens, int H, int dk, int dv,
                             const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, int num_seqs,
                             float lower_bound, float* M_out, float* N_out, void* workspace, size_t workspace_bytes,
                             void* hip_stream)
{
    REQUIRE(valid_dtype(in_dtype), KDA_ERR_INVALID_ARG, "kda_prefill_segment_maps: bad dtype");
    REQUIRE(in_dtype == KDA_BF16, KDA_ERR_UNSUPPORTED,
            "kda_prefill_segment_maps: only bfloat16 inputs are supported (the two-pass form)");
    REQUIRE(num_tokens >= 0 && H >= 1, KDA_ERR_INVALID_ARG, "kda_prefill_segment_maps: bad num_tokens or H");
    REQUIRE(dk == 128 && dv == 128, KDA_ERR_UNSUPPORTED,
            "kda_prefill_segment_maps: only dk = dv = 128 is supported (got %d, %d)", dk, dv);
    if (int rc = check_lower_bound("kda_prefill_segment_maps", lower_bound, true); rc != KDA_OK) return rc;
    REQUIRE(M_out && N_out, KDA_ERR_INVALID_ARG, "kda_prefill_segment_maps: null M_out or N_out");
    REQUIRE(num_tokens == 0 || (k && v && g && beta), KDA_ERR_INVALID_ARG,
            "kda_prefill_segment_maps: null tensor pointer");
    REQUIRE(workspace, KDA_ERR_WORKSPACE, "kda_prefill_segment_maps: a workspace is required");
    for (const void* p : {k, v, g, beta, (const void*)M_out, (const void*)N_out, (const void*)workspace})
        REQUIRE(!p || aligned16(p), KDA_ERR_INVALID_ARG, "kda_prefill_segment_maps: pointers must be 16-byte aligned");
    int64_t seq_len = 0;
    int rc = check_cu(cu_seqlens_dev, cu_seqlens_host, num_seqs, num_tokens, &seq_len);
    if (rc != KDA_OK) return rc;
    REQUIRE((int64_t)num_seqs * H * 4 <= 0x7fffffff, KDA_ERR_INVALID_ARG, "kda_prefill_segment_maps: num_seqs*H too large");
    const int64_t units = (int64_t)num_seqs * H;
    int64_t max_len = seq_len;
    if (cu_seqlens_host)
        for (int n = 0; n < num_seqs; ++n)
            max_len = std::max<int64_t>(max_len, (int64_t)cu_seqlens_host[n + 1] - cu_seqlens_host[n]);
    const int64_t max_chunks = (max_len + kChunk - 1) / kChunk;
    const size_t slot = prefill_split_slot_bytes();
    const size_t whole = (size_t)(units * std::max<int64_t>(max_chunks, 1)) * slot;
    const size_t least = (size_t)units * slot + state_carry_bytes(units);
    REQUIRE(workspace_bytes >= std::min(whole, least), KDA_ERR_WORKSPACE,
            "kda_prefill_segment_maps: workspace of at least %zu bytes required (got %zu)", std::min(whole, least),
            workspace_bytes);
    const size_t T = (size_t)num_tokens, mbytes = (size_t)units * 128 * 128 * 4;
    const Range rM = rng(M_out, mbytes), rN = rng(N_out, mbytes), rws = rng(workspace, workspace_bytes);
    REQUIRE(!overlap(rM, rN), KDA_ERR_INVALID_ARG, "kda_prefill_segment_maps: M_out overlaps N_out");
    for (const Range& r : {rng(k, T * H * 256), rng(v, T * H * 256), rng(g, T * H * 256), rng(beta, T * H * 2), rws})
        REQUIRE(!overlap(r, rM) && !overlap(r, rN), KDA_ERR_INVALID_ARG,
                "kda_prefill_segment_maps: M_out or N_out overlaps an input or the workspace");
    for (const Range& r : {rng(k, T * H * 256), rng(v, T * H * 256), rng(g, T * H * 256), rng(beta, T * H * 2)})
        REQUIRE(!overlap(r, rws), KDA_ERR_INVALID_ARG, "kda_prefill_segment_maps: workspace overlaps an input");

    PrefillArgs a{};
    a.q = k;  // never read: the map pass forms no query side
    a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.cu_seqlens = cu_seqlens_dev; a.seq_len = seq_len;
    a.sT = N_out; a.map_M = M_out;
    a.num_seqs = num_seqs; a.H = H; a.scale = 1.0f; a.lower_bound = lower_bound;
    a.in_dtype = BF16; a.out_dtype = F32;
    return hip_status(launch_prefill_split(a, workspace, workspace_bytes, max_chunks, cu_seqlens_host,
                                           static_cast<hipStream_t>(hip_stream)),
                      "kda_prefill_segment_maps");
}

int kda_affine_apply(const float* M, const float* X, const float* N, float* Y, int64_t count, int dk, int dv,
                     void* hip_stream)
{
    REQUIRE(dk == 128 && dv == 128, KDA_ERR_UNSUPPORTED,
            "kda_affine_apply: only dk = dv = 128 is supported (got %d, %d)", dk, dv);
    REQUIRE(count >= 0, KDA_ERR_INVALID_ARG, "kda_affine_apply: negative count");
    if (count == 0) return KDA_OK;
    REQUIRE(M && X && Y, KDA_ERR_INVALID_ARG, "kda_affine_apply: null M, X or Y");
    for (const void* p : {(const void*)M, (const void*)X, (const void*)N, (const void*)Y})
        REQUIRE(!p || aligned16(p), KDA_ERR_INVALID_ARG, "kda_affine_apply: pointers must be 16-byte aligned");
    const size_t bytes = (size_t)count * 128 * 128 * 4;
    const Range rY = rng(Y, bytes), rN = rng(N, N ? bytes : 0);
    REQUIRE(!overlap(rY, rng(M, bytes)) && !overlap(rY, rng(X, bytes)), KDA_ERR_INVALID_ARG,
            "kda_affine_apply: Y overlaps M or X");
    REQUIRE(!overlap(rY, rN) || N == Y, KDA_ERR_INVALID_ARG,
            "kda_affine_apply: Y and N overlap without being the same buffer");
    return hip_status(launch_affine_apply(M, X, N, Y, count, static_cast<hipStream_t>(hip_stream)),
                      "kda_affine_apply");
}

// ---------------------------------------------------------------- GEMM
int kda_gemm(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
             int64_t M, int64_t N, int64_t K, kda_dtype ab_dtype, kda_dtype c_dtype,
             void* hip_stream)
{
    REQUIRE(A && B && C, KDA_ERR_INVALID_ARG, "kda_gemm: null pointer");
    REQUIRE(valid_dtype(ab_dtype) && valid_dtype(c_dtype), KDA_ERR_INVALID_ARG, "kda_gemm: bad dtype");
    REQUIRE(ab_dtype == KDA_BF16, KDA_ERR_UNSUPPORTED, "kda_gemm: only bfloat16 A and B are supported");
    REQUIRE(M >= 1 && N >= 1 && K >= 8, KDA_ERR_INVALID_ARG, "kda_gemm: bad sizes");
    REQUIRE(K % 8 == 0, KDA_ERR_UNSUPPORTED, "kda_gemm: K must be a multiple of 8");
    REQUIRE(lda >= K && ldb >= K && ldc >= N && lda % 8 == 0 && ldb % 8 == 0 && ldc % 4 == 0,
            KDA_ERR_INVALID_ARG, "kda_gemm: lda, ldb >= K (multiples of 8), ldc >= N (multiple of 4)");
    for (const void* p : {A, B, (const void*)C})
        REQUIRE(aligned16(p), KDA_ERR_INVALID_ARG, "kda_gemm: pointers must be 16-byte aligned");
    const Range rc = rng(C, ((size_t)(M - 1) * ldc + N) * esize(c_dtype));
    REQUIRE(!overlap(rc, rng(A, ((size_t)(M - 1) * lda + K) * 2)) && !overlap(rc, rng(B, ((size_t)(N - 1) * ldb + K) * 2)),
            KDA_ERR_INVALID_ARG, "kda_gemm: C overlaps A or B");
    GemmArgs a{A, B, C, lda, ldb, ldc, M, N, K, (DType)c_dtype};
    return hip_status(launch_gemm(a, static_cast<hipStream_t>(hip_stream)), "kda_gemm");
}

}  // extern "C"
