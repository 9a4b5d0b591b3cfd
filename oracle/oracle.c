/*
 * CPU oracle, fp32 decision part.  TEST INFRASTRUCTURE ONLY: the product path
 * (the HIP library and its Python binding) never links, loads or calls this.
 * It is built by oracle/build.py with gcc -O2 -ffp-contract=off and loaded by
 * the tests, by __graft_entry__.smoke() and by bench.py's cpu_baseline leg.
 *
 * What lives here: the steps where floating point decides an integer, i.e.
 * which experts a token is routed to.  They run in fp32, the precision the
 * GPU kernel takes the same decision in, so that given the same fp32 logits
 * both sides must pick the same experts bit for bit.  Everything else of the
 * oracle (logits, weights, expert FFN, combine, shuffle) is fp64 numpy in
 * oracle/moe_oracle.py.
 *
 * Sources.  The pages (Sem-MoE summaries, "Semantic Parallelism: Redefining
 * Efficient MoE Inference via Model-Data Co-Scheduling") say only that each
 * token activates a few experts chosen by the gate (technical summary §1) and
 * that the gate's columns are shuffled to place experts (technical overview
 * §2.2A).  The gate function, top-k rule and tie-break are not on the pages;
 * the readings used (documented with the oracle) are:
 *   - top-k orders experts by (key descending, ORIGINAL expert id ascending);
 *   - softmax gates select on the logit itself (softmax is monotone);
 *   - the sigmoid gate with per-expert bias selects on sigmoid(l) + b and, when
 *     grouped, first keeps topk_rgroups routing groups (contiguous blocks of
 *     original ids) by the sum of their rgroup_topn largest keys, summed in
 *     descending order, ties to the lower group id.
 *
 * exp: sigmoid needs exp, and its result decides the selection, so both sides
 * implement the same published method rather than a vendor libm:
 * Cody-Waite additive range reduction (W. J. Cody and W. Waite, "Software
 * Manual for the Elementary Functions", 1980): n = rint(x*log2(e)),
 * r = x - n*ln2 (ln2 split in a high and a low fp32 part, each step one fused
 * multiply-add), then exp(r) by the degree-7 Taylor polynomial in Horner form
 * with fused multiply-adds, then an exact scaling by 2^n.  Defined on
 * [-87, 88] (normal results); below it returns 0, above it +inf.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef union { float f; uint32_t u; } f32u;

static float pow2i(int n) /* 2^n for -126 <= n <= 127 */
{
    f32u v;
    v.u = (uint32_t)(n + 127) << 23;
    return v.f;
}

float oracle_expf(float x)
{
    /* ln 2 = 0.6931471805599453094...; hi = ln2 rounded to fp32, lo = the
     * fp32 rounding of the remainder; log2(e) rounded to fp32. */
    const float ln2_hi = (float)0.69314718055994530942;
    const float ln2_lo = (float)(0.69314718055994530942 - (double)(float)0.69314718055994530942);
    const float log2e = (float)1.44269504088896340736;
    /* Taylor coefficients 1/j!, j = 0..7 */
    const float c[8] = {1.0f, 1.0f, (float)(1.0 / 2.0), (float)(1.0 / 6.0),
                        (float)(1.0 / 24.0), (float)(1.0 / 120.0),
                        (float)(1.0 / 720.0), (float)(1.0 / 5040.0)};
    if (x != x) return x;
    if (x < -87.0f) return 0.0f;
    if (x > 88.0f) return INFINITY;
    float n = rintf(x * log2e);
    float r = fmaf(-n, ln2_hi, x);
    r = fmaf(-n, ln2_lo, r);
    float p = c[7];
    for (int j = 6; j >= 0; --j) p = fmaf(p, r, c[j]);
    return p * pow2i((int)n);
}

float oracle_sigmoidf(float l)
{
    float e = oracle_expf(-l);
    float d = 1.0f + e;
    return 1.0f / d;
}

void oracle_expf_array(int64_t n, const float* x, float* y)
{
    for (int64_t i = 0; i < n; ++i) y[i] = oracle_expf(x[i]);
}

/* key[t,e] = sigmoid(logit[t,e]) + bias[e]  (fp32, original expert order);
 * sig[t,e] = sigmoid(logit[t,e]).  bias may be NULL (treated as 0). */
void oracle_sigmoid_keys(int T, int E, const float* logit, const float* bias,
                         float* key, float* sig)
{
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            float s = oracle_sigmoidf(logit[(int64_t)t * E + e]);
            sig[(int64_t)t * E + e] = s;
            key[(int64_t)t * E + e] = bias ? s + bias[e] : s;
        }
}

/* a beats b: larger key, or equal key and lower original id */
static int better(float ka, int ia, float kb, int ib)
{
    return ka > kb || (ka == kb && ia < ib);
}

/*
 * Top-k selection for T tokens over E experts in ORIGINAL order.
 *   key      [T,E] fp32 selection keys
 *   k_tok    [T]   per-token k (NULL: every token takes k_max)
 *   sel      [T,k_max] out: chosen original ids in selection order, -1 padding
 *   n_rgroups, topk_rgroups, rgroup_topn: group-limited routing; n_rgroups <= 1
 *            or topk_rgroups >= n_rgroups means plain top-k.  Routing group of
 *            expert e is e / (E / n_rgroups).
 * Returns 0, or -1 on bad arguments.
 */
int oracle_select(int T, int E, const float* key, const int32_t* k_tok, int k_max,
                  int n_rgroups, int topk_rgroups, int rgroup_topn, int32_t* sel)
{
    if (T < 0 || E <= 0 || k_max <= 0 || k_max > E || E > 4096) return -1;
    int grouped = n_rgroups > 1 && topk_rgroups < n_rgroups;
    if (grouped && (E % n_rgroups != 0 || rgroup_topn <= 0 || rgroup_topn > E / n_rgroups || n_rgroups > 256))
        return -1;
    unsigned char taken[4096];
    unsigned char allowed[4096];
    for (int t = 0; t < T; ++t) {
        const float* kr = key + (int64_t)t * E;
        int kt = k_tok ? k_tok[t] : k_max;
        if (kt < 0 || kt > k_max) return -1;
        for (int e = 0; e < E; ++e) allowed[e] = 1;
        if (grouped) {
            int gsize = E / n_rgroups;
            float score[256];
            unsigned char kept[256];
            for (int g = 0; g < n_rgroups; ++g) {
                /* sum of the rgroup_topn largest keys, largest first */
                for (int e = 0; e < gsize; ++e) taken[e] = 0;
                float s = 0.0f;
                for (int j = 0; j < rgroup_topn; ++j) {
                    int best = -1;
                    for (int e = 0; e < gsize; ++e) {
                        if (taken[e]) continue;
                        if (best < 0 || kr[g * gsize + e] > kr[g * gsize + best]) best = e;
                    }
                    taken[best] = 1;
                    s = (j == 0) ? kr[g * gsize + best] : s + kr[g * gsize + best];
                }
                score[g] = s;
                kept[g] = 0;
            }
            for (int j = 0; j < topk_rgroups; ++j) {
                int best = -1;
                for (int g = 0; g < n_rgroups; ++g) {
                    if (kept[g]) continue;
                    if (best < 0 || better(score[g], g, score[best], best)) best = g;
                }
                kept[best] = 1;
            }
            for (int e = 0; e < E; ++e) allowed[e] = kept[e / gsize];
        }
        for (int e = 0; e < E; ++e) taken[e] = 0;
        for (int j = 0; j < k_max; ++j) {
            if (j >= kt) { sel[(int64_t)t * k_max + j] = -1; continue; }
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e] || !allowed[e]) continue;
                if (best < 0 || better(kr[e], e, kr[best], best)) best = e;
            }
            if (best < 0) return -1; /* fewer allowed experts than k */
            taken[best] = 1;
            sel[(int64_t)t * k_max + j] = best;
        }
    }
    return 0;
}
