// Host-side speedup model of speculative decoding, fed by measured times.
//
// LLM Primer ch. 9, section 9.3: a speculative step's speedup is the expected
// number of tokens it emits over (T_draft / T_decode + 1 + alpha * N), alpha
// the verification overhead per candidate position; the alpha * N term sets a
// best N, and 1 / alpha bounds the speedup as acceptance approaches 1. A
// chain of N candidates accepted with probability p each emits
// sum_{i<=N} p^i tokens on average (jisaku.com glossary, linear-speculation
// closed form). alpha is read off verification times T(N) measured on this
// GPU: the least-squares slope of T(N) / T(1) - 1 against N - 1.

#include <cmath>

#include "common.h"

extern "C" double tav_model_speedup(double expected_emitted, double draft_ratio, double alpha,
                                    int32_t n)
{
    const double den = draft_ratio + 1.0 + alpha * (double)n;
    if (n < 0 || !(expected_emitted >= 0.0) || !(draft_ratio >= 0.0) || !(alpha >= 0.0) ||
        !(den > 0.0) || !std::isfinite(den))
        return NAN;
    return expected_emitted / den;
}

extern "C" int32_t tav_best_chain_length(double p, double draft_ratio, double alpha,
                                         int32_t n_max, double *speedup_out)
{
    if (!(p >= 0.0 && p <= 1.0) || !(draft_ratio >= 0.0) || !(alpha >= 0.0) || n_max < 1 ||
        !std::isfinite(draft_ratio) || !std::isfinite(alpha))
        return 0;
    int32_t best = 0;
    double best_s = -INFINITY;
    double emitted = 1.0, pk = 1.0;   // sum_{i<=n} p^i, p^n
    for (int32_t n = 1; n <= n_max; ++n) {
        pk *= p;
        emitted += pk;
        const double s = emitted / (draft_ratio + 1.0 + alpha * (double)n);
        if (s > best_s) {
            best = n;
            best_s = s;
        }
    }
    if (speedup_out)
        *speedup_out = best_s;
    return best;
}

extern "C" double tav_fit_alpha(const int32_t *n, const double *t_us, int32_t count)
{
    if (!n || !t_us || count < 2 || n[0] != 1 || !(t_us[0] > 0.0))
        return NAN;
    double sxy = 0.0, sxx = 0.0;
    for (int32_t k = 0; k < count; ++k) {
        if (n[k] < 1 || !(t_us[k] > 0.0) || !std::isfinite(t_us[k]))
            return NAN;
        const double x = (double)(n[k] - 1);
        sxy += x * (t_us[k] / t_us[0] - 1.0);
        sxx += x * x;
    }
    return sxx > 0.0 ? sxy / sxx : NAN;
}

// The same model with a whole decode step as its baseline, at batch B: a
// layer's linear projections and the vocabulary head by their roofline
// (bf16 weights read once, or 2 FLOP per weight per token), one layer's
// attention and the walk as measured. The verification pass scores B*n
// tokens where a decode step scores B, which is why the speedup falls as the
// batch grows (the yuuk.io wiki's observation).
namespace {

double linear_us(double params, double tokens, double hbm_gbs, double mfma_tflops)
{
    const double t_mem = 2.0 * params / (hbm_gbs * 1e3);
    const double t_mac = 2.0 * params * tokens / (mfma_tflops * 1e6);
    return t_mem > t_mac ? t_mem : t_mac;
}

} // namespace

extern "C" double tav_verify_speedup(double expected_emitted, double draft_ratio, int32_t layers,
                                     double layer_params, double head_params, int32_t batch,
                                     int32_t n, double attn_verify_us, double sampler_verify_us,
                                     double attn_decode_us, double sampler_decode_us,
                                     double hbm_gbs, double mfma_tflops, double *out)
{
    const double args[] = {expected_emitted, draft_ratio, layer_params, head_params,
                           attn_verify_us, sampler_verify_us, attn_decode_us, sampler_decode_us};
    for (double v : args)
        if (!(v >= 0.0) || !std::isfinite(v))
            return NAN;
    if (layers < 1 || batch < 1 || n < 1 || !(hbm_gbs > 0.0) || !(mfma_tflops > 0.0))
        return NAN;
    const double t_dec = layers * (linear_us(layer_params, batch, hbm_gbs, mfma_tflops) +
                                   attn_decode_us) +
                         linear_us(head_params, batch, hbm_gbs, mfma_tflops) + sampler_decode_us;
    const double t_ver = layers * (linear_us(layer_params, (double)batch * n, hbm_gbs,
                                             mfma_tflops) +
                                   attn_verify_us) +
                         linear_us(head_params, (double)batch * n, hbm_gbs, mfma_tflops) +
                         sampler_verify_us;
    if (!(t_dec > 0.0))
        return NAN;
    const double alpha = (t_ver / t_dec - 1.0) / n;
    if (out) {
        out[0] = alpha;
        out[1] = t_dec;
        out[2] = t_ver;
    }
    return expected_emitted / (draft_ratio + 1.0 + alpha * n);
}
