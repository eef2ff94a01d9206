/*
 * CPU ORACLE for the Switch FFN layer forward pass -- TEST INFRASTRUCTURE.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load or call this library.  The HIP product path never links or calls it,
 * and it includes none of the product's headers: the two share no code.
 *
 * It is the plain definition of what the layer computes, evaluated in double
 * precision from the exact input values (bf16 and fp32 inputs widen exactly),
 * one step after another, with no blocking, fusion or reordering beyond what
 * each definition states.  OpenMP only splits independent tokens (or
 * independent experts) across threads; every sum keeps its natural order.
 *
 * Pages cited (all describe the Switch Transformers paper, Fedus, Zoph and
 * Shazeer):
 *   [MS]  "Switch Transformer - Scaling to Trillion Parameter Models with Simple
 *          and Efficient Sparsity" (Incredible.AI blog): sections "Expert
 *          Capacity", "Differentiable Load Balancing Loss", "MoE Layer".
 *   [KB]  "Switch Transformerとは？巨大モデルを効率化するMoE" (kasblo
 *          explainer): sections "Top-1 Routingを数式で追う",
 *          "tokenをExpertへ送って戻すforward pass", "Expert Capacityは
 *          tokenの受付上限", "16 token、4 Expertで考える",
 *          "補助負荷分散lossは何を均等にするのか",
 *          "Routerだけfloat32で計算するSelective Precision".
 *   [BH]  "Switch Transformer by Hand" (byhand.ai): walkthrough steps [5]-[13].
 *   [LP]  "精读 06 | Switch Transformers" (llm-papers-study close reading):
 *          sections 3.1 (router logits and softmax), 3.2 (switch routing),
 *          3.3 (load-balancing loss), 3.4 (capacity factor, dropped tokens),
 *          part 六 (architecture diagram).
 *
 * Readings taken where the pages are silent or disagree (listed with reasons
 * in the design notes):
 *   - capacity C = ceil(c * T / N) with T = every token of the call;
 *   - argmax over the logits, lowest index on an exact tie;
 *   - f_i counts tokens before the capacity cut;
 *   - the expert FFN is relu(x W_in^T) W_out^T without biases;
 *   - out = x + gate * E(x) inside the layer; a dropped token leaves unchanged.
 *
 * Top-k routing (the MoE routing the Switch layer simplifies; [LP 3.1] and
 * [MS] "Mixture of Experts Routing") follows further down, with its own
 * readings.
 *
 * Parity pins: every function here is pinned by the -m "not gpu" tests
 * (worked examples of the pages, closed forms, brute force, a library matmul
 * for the dense special case).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define NT(n) ((n) > 0 ? (n) : 1)

/*
 * O-4  Expert capacity.  [LP 3.4] expert capacity = (tokens per batch /
 * number of experts) x capacity factor; [KB "Expert Capacityはtokenの受付上限"]
 * rounds it to an integer.  Reading: round up, over all T tokens of the call.
 * A positive override replaces the formula (worked examples that print C).
 */
int64_t oracle_capacity(int64_t T, int64_t N, double c, int64_t capacity_override) {
  if (capacity_override > 0) return capacity_override;
  if (N <= 0) return 0;
  double v = ceil((c * (double)T) / (double)N);
  return v < 0.0 ? 0 : (int64_t)v;
}

/*
 * O-1  Router logits h(x) = W_r . x  ([LP 3.1]; [MS] "Expert Capacity" recap of
 * MoE routing), plus an optional per-expert bias.  W_r is [N, d] (one row per
 * expert), x is [T, d]; h is [T, N].  Accumulated in double in k order.
 */
void oracle_logits(const float* x, const float* W_r, const float* b_r, int64_t T, int64_t d,
                   int64_t N, double* h, int nthreads) {
#pragma omp parallel for schedule(static) num_threads(NT(nthreads))
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t i = 0; i < N; ++i) {
      double acc = 0.0;
      for (int64_t k = 0; k < d; ++k) acc += (double)x[t * d + k] * (double)W_r[i * d + k];
      if (b_r) acc += (double)b_r[i];
      h[t * N + i] = acc;
    }
  }
}

/* Logits of selected tokens only (large workloads are checked on samples). */
void oracle_logits_rows(const float* x_rows /* [n, d] */, int64_t n, const float* W_r,
                        const float* b_r, int64_t d, int64_t N, double* h /* [n, N] */,
                        int nthreads) {
  oracle_logits(x_rows, W_r, b_r, n, d, N, h, nthreads);
}

/*
 * O-2, O-3  Softmax gate and top-1 choice for one token.
 * [LP 3.1] p_i(x) = exp(h_i) / sum_j exp(h_j); [LP 3.2] the chosen expert is
 * argmax_i p_i(x) and the output is scaled by p of that expert; [KB
 * "Top-1 Routingを数式で追う"] the router scores every expert and runs one.
 * The max is subtracted before exponentiating (same value in exact
 * arithmetic).  Returns i*, writes gate = p_{i*}, max m and sum S.
 */
static int32_t route_token(const double* h, int64_t N, double* gate, double* m_out, double* S_out) {
  int32_t best = 0;
  double m = h[0];
  for (int64_t i = 1; i < N; ++i)
    if (h[i] > m) { m = h[i]; best = (int32_t)i; }
  double S = 0.0;
  for (int64_t i = 0; i < N; ++i) S += exp(h[i] - m);
  *gate = exp(h[best] - m) / S;
  *m_out = m;
  *S_out = S;
  return best;
}

/*
 * O-2 .. O-6  Routing stage of the layer, applied to given logits h [T, N]
 * (the oracle's own, or the GPU's fp32 logits widened to double).
 *
 *   expert_idx[t], gate[t]         top-1 and its softmax probability
 *   position[t]                    rank of t among the tokens routed to the
 *                                  same expert, in token order
 *                                  ([MS] "MoE Layer": an expert keeps the first
 *                                  `capacity` of its tokens in flattened token
 *                                  order; [KB "16 token、4 Expertで考える"];
 *                                  [BH] step 7: Z5 arrives after Expert C is
 *                                  full)
 *   drop[t] = position[t] >= C     overflow tokens skip the expert
 *                                  ([LP 3.4]; [KB "Expert Capacityは..."])
 *   load[e]                        tokens routed to e, before the capacity cut
 *   P[e] = (1/T) sum_t p_e(t)      mean router probability ([LP 3.3])
 *   aux = alpha N sum_e f_e P_e,   f_e = load[e] / T ([LP 3.3]; [KB
 *                                  "補助負荷分散lossは何を均等にするのか"])
 *
 * P_out may be NULL.  Returns the capacity C.
 */
int64_t oracle_route(const double* h, int64_t T, int64_t N, double c, int64_t capacity_override,
                     double alpha, int32_t* expert_idx, double* gate, int32_t* position,
                     uint8_t* drop, int32_t* load, double* P_out, double* aux, int nthreads) {
  int64_t C = oracle_capacity(T, N, c, capacity_override);
  double* m = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  double* S = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  double* P = (double*)calloc((size_t)(N > 0 ? N : 1), sizeof(double));

#pragma omp parallel for schedule(static) num_threads(NT(nthreads))
  for (int64_t t = 0; t < T; ++t)
    expert_idx[t] = route_token(h + t * N, N, &gate[t], &m[t], &S[t]);

  /* one sequential pass in token order */
  for (int64_t e = 0; e < N; ++e) load[e] = 0;
  for (int64_t t = 0; t < T; ++t) {
    int32_t e = expert_idx[t];
    position[t] = load[e];
    load[e] += 1;
    drop[t] = (uint8_t)((int64_t)position[t] >= C);
  }

  /* P_e = (1/T) sum over tokens of p_e(t); each expert's sum runs in token order */
#pragma omp parallel for schedule(static) num_threads(NT(nthreads))
  for (int64_t e = 0; e < N; ++e) {
    double acc = 0.0;
    for (int64_t t = 0; t < T; ++t) acc += exp(h[t * N + e] - m[t]) / S[t];
    P[e] = T > 0 ? acc / (double)T : 0.0;
  }

  double sum = 0.0;
  for (int64_t e = 0; e < N; ++e) {
    double f = T > 0 ? (double)load[e] / (double)T : 0.0;
    sum += f * P[e];
  }
  *aux = alpha * (double)N * sum;
  if (P_out) memcpy(P_out, P, sizeof(double) * (size_t)N);
  free(m);
  free(S);
  free(P);
  return C;
}

/*
 * O-7  One expert's FFN on one token: E = W_out . relu(W_in . x)
 * (the dense FFN the Switch layer replaces, [KB "TransformerのどこへSwitch
 * layerが入るのか"]; no biases).  W_in is [F, d], W_out is [d, F].
 * Double accumulation, no intermediate rounding.
 */
static void expert_ffn(const float* x, const float* W_in, const float* W_out, int64_t d, int64_t F,
                       double* u /* [F] scratch */, double* E /* [d] */) {
  for (int64_t j = 0; j < F; ++j) {
    double acc = 0.0;
    for (int64_t k = 0; k < d; ++k) acc += (double)W_in[j * d + k] * (double)x[k];
    u[j] = acc > 0.0 ? acc : 0.0;
  }
  for (int64_t i = 0; i < d; ++i) {
    double acc = 0.0;
    for (int64_t j = 0; j < F; ++j) acc += (double)W_out[i * F + j] * u[j];
    E[i] = acc;
  }
}

/*
 * O-7, O-8  Output row of one token.  [LP 3.2] y = p_{i*}(x) E_{i*}(x);
 * part 六 adds the residual; [LP 3.4] and [BH] step 13: a dropped token is
 * passed through unchanged.  `W_in_e`/`W_out_e` are the chosen expert's
 * weights.  out[k] = x[k] + gate * E[k] (kept) or x[k] (dropped).
 */
void oracle_token_output(const float* x, int32_t dropped, double gate, const float* W_in_e,
                         const float* W_out_e, int64_t d, int64_t F, double* out,
                         double* E_out /* [d] or NULL: the expert output itself */) {
  if (dropped) {
    for (int64_t k = 0; k < d; ++k) out[k] = (double)x[k];
    if (E_out) for (int64_t k = 0; k < d; ++k) E_out[k] = 0.0;
    return;
  }
  double* u = (double*)malloc(sizeof(double) * (size_t)F);
  double* E = (double*)malloc(sizeof(double) * (size_t)d);
  expert_ffn(x, W_in_e, W_out_e, d, F, u, E);
  for (int64_t k = 0; k < d; ++k) out[k] = (double)x[k] + gate * E[k];
  if (E_out) memcpy(E_out, E, sizeof(double) * (size_t)d);
  free(u);
  free(E);
}

/*
 * Combine stage for a whole call, given a routing (expert_idx, gate, drop):
 * O-7 and O-8 for every token.  W_in is [N, F, d], W_out is [N, d, F].
 * E_out [T, d] (may be NULL) receives the expert output of kept tokens and 0
 * for dropped ones.
 */
void oracle_combine(const float* x, const int32_t* expert_idx, const double* gate,
                    const uint8_t* drop, const float* W_in, const float* W_out, int64_t T,
                    int64_t d, int64_t F, double* out, double* E_out, int nthreads) {
#pragma omp parallel for schedule(dynamic, 4) num_threads(NT(nthreads))
  for (int64_t t = 0; t < T; ++t) {
    int64_t e = expert_idx[t];
    oracle_token_output(x + t * d, drop[t], gate[t], W_in + e * F * d, W_out + e * d * F, d, F,
                        out + t * d, E_out ? E_out + t * d : NULL);
  }
}

/*
 * The whole layer: O-1 logits, O-2..O-6 routing, O-7..O-8 combine.
 * Returns the capacity C.  h [T, N] is written (caller storage).
 */
int64_t oracle_forward(const float* x, const float* W_r, const float* b_r, const float* W_in,
                       const float* W_out, int64_t T, int64_t d, int64_t F, int64_t N, double c,
                       int64_t capacity_override, double alpha, double* h, int32_t* expert_idx,
                       double* gate, int32_t* position, uint8_t* drop, int32_t* load, double* P,
                       double* aux, double* out, double* E_out, int nthreads) {
  oracle_logits(x, W_r, b_r, T, d, N, h, nthreads);
  int64_t C = oracle_route(h, T, N, c, capacity_override, alpha, expert_idx, gate, position, drop,
                           load, P, aux, nthreads);
  oracle_combine(x, expert_idx, gate, drop, W_in, W_out, T, d, F, out, E_out, nthreads);
  return C;
}

/* ------------------------------------------------------------------------
 * Top-k routing, the MoE routing that the Switch layer reduces to k = 1.
 * [LP 3.1]: the router scores all N experts, p = softmax(h), and the output
 * is the sum over the selected set T of p_i(x) E_i(x), where T holds the K
 * experts with the highest scores (classic MoE: usually K = 2); its hospital
 * illustration weights the two chosen departments by 0.6 and 0.3.  [MS]
 * "Mixture of Experts Routing" (MoELayer code): torch.topk over the softmax
 * probabilities, each chosen expert's output weighted by its probability.
 * [LP 3.2], point (2): with one expert per token the capacity can at least be
 * halved, i.e. k choices per token need k times the top-1 capacity.
 *
 * Readings (the pages do not give these steps):
 *   - the k experts are the k largest logits, ties to the lower index, chosen
 *     one after another (the best, then the best of the rest, ...);
 *   - gates are the full-softmax probabilities of the chosen experts, not
 *     renormalised over the chosen set;
 *   - capacity C = ceil(k c T / N), or the override;
 *   - assignments take positions in the order (t, j): token order, and within
 *     a token its choices in rank order; each assignment is dropped on its own
 *     when its position reaches C;
 *   - out = x + sum over kept choices of gate_j E_{e_j}(x); a token with all
 *     choices dropped leaves unchanged;
 *   - the loss keeps its form with f_e = load_e / (k T), load_e counting all
 *     assignments before the capacity cut (so f sums to 1 and a uniform load
 *     still gives alpha).
 * With k = 1 every one of these is the top-1 definition above.
 * ------------------------------------------------------------------------ */

int64_t oracle_capacity_topk(int64_t T, int64_t N, int64_t k, double c,
                             int64_t capacity_override) {
  if (capacity_override > 0) return capacity_override;
  if (N <= 0) return 0;
  double v = ceil(((double)k * c * (double)T) / (double)N);
  return v < 0.0 ? 0 : (int64_t)v;
}

/* The k best experts of one token by logit (ties: lower index first), their
 * softmax probabilities, and the row's max and sum for P. */
static void route_token_topk(const double* h, int64_t N, int64_t k, int32_t* idx, double* gate,
                             double* m_out, double* S_out) {
  double m = h[0];
  for (int64_t i = 1; i < N; ++i)
    if (h[i] > m) m = h[i];
  double S = 0.0;
  for (int64_t i = 0; i < N; ++i) S += exp(h[i] - m);
  for (int64_t j = 0; j < k; ++j) {
    int32_t best = -1;
    for (int64_t i = 0; i < N; ++i) {
      int taken = 0;
      for (int64_t q = 0; q < j; ++q) taken |= (idx[q] == (int32_t)i);
      if (taken) continue;
      if (best < 0 || h[i] > h[best]) best = (int32_t)i;
    }
    idx[j] = best;
    gate[j] = exp(h[best] - m) / S;
  }
  *m_out = m;
  *S_out = S;
}

/*
 * Top-k routing stage on given logits h [T, N].  Outputs are [T, k] row-major
 * (expert_idx, gate, position, drop) and load [N]; P_out [N] may be NULL.
 * Returns C.  Requires 1 <= k <= N.
 */
int64_t oracle_route_topk(const double* h, int64_t T, int64_t N, int64_t k, double c,
                          int64_t capacity_override, double alpha, int32_t* expert_idx,
                          double* gate, int32_t* position, uint8_t* drop, int32_t* load,
                          double* P_out, double* aux, int nthreads) {
  int64_t C = oracle_capacity_topk(T, N, k, c, capacity_override);
  double* m = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  double* S = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  double* P = (double*)calloc((size_t)(N > 0 ? N : 1), sizeof(double));

#pragma omp parallel for schedule(static) num_threads(NT(nthreads))
  for (int64_t t = 0; t < T; ++t)
    route_token_topk(h + t * N, N, k, expert_idx + t * k, gate + t * k, &m[t], &S[t]);

  /* one sequential pass over the assignments in (token, choice) order */
  for (int64_t e = 0; e < N; ++e) load[e] = 0;
  for (int64_t a = 0; a < T * k; ++a) {
    int32_t e = expert_idx[a];
    position[a] = load[e];
    load[e] += 1;
    drop[a] = (uint8_t)((int64_t)position[a] >= C);
  }

#pragma omp parallel for schedule(static) num_threads(NT(nthreads))
  for (int64_t e = 0; e < N; ++e) {
    double acc = 0.0;
    for (int64_t t = 0; t < T; ++t) acc += exp(h[t * N + e] - m[t]) / S[t];
    P[e] = T > 0 ? acc / (double)T : 0.0;
  }

  double sum = 0.0;
  for (int64_t e = 0; e < N; ++e) {
    double f = T > 0 ? (double)load[e] / ((double)k * (double)T) : 0.0;
    sum += f * P[e];
  }
  *aux = alpha * (double)N * sum;
  if (P_out) memcpy(P_out, P, sizeof(double) * (size_t)N);
  free(m);
  free(S);
  free(P);
  return C;
}

/*
 * Top-k combine: out[t] = x[t] + sum over kept j of gate[t,j] E_{e[t,j]}(x[t])
 * ([LP 3.1] weighted sum of the selected experts, plus the residual of part
 * 六).  E_out [T, k, d] (may be NULL) receives each choice's expert output, 0
 * for a dropped choice.
 */
void oracle_combine_topk(const float* x, const int32_t* expert_idx, const double* gate,
                         const uint8_t* drop, const float* W_in, const float* W_out, int64_t T,
                         int64_t k, int64_t d, int64_t F, double* out, double* E_out,
                         int nthreads) {
#pragma omp parallel for schedule(dynamic, 4) num_threads(NT(nthreads))
  for (int64_t t = 0; t < T; ++t) {
    double* u = (double*)malloc(sizeof(double) * (size_t)F);
    double* E = (double*)malloc(sizeof(double) * (size_t)d);
    const float* xt = x + t * d;
    double* o = out + t * d;
    for (int64_t q = 0; q < d; ++q) o[q] = (double)xt[q];
    for (int64_t j = 0; j < k; ++j) {
      const int64_t a = t * k + j;
      double* Ea = E_out ? E_out + a * d : NULL;
      if (drop[a]) {
        if (Ea) for (int64_t q = 0; q < d; ++q) Ea[q] = 0.0;
        continue;
      }
      const int64_t e = expert_idx[a];
      expert_ffn(xt, W_in + e * F * d, W_out + e * d * F, d, F, u, E);
      for (int64_t q = 0; q < d; ++q) o[q] += gate[a] * E[q];
      if (Ea) memcpy(Ea, E, sizeof(double) * (size_t)d);
    }
    free(u);
    free(E);
  }
}

/* ------------------------------------------------------------------------
 * Backward pass of the top-1 layer: gradients of L with respect to x, W_r,
 * b_r, W_in and W_out, given G = dL/dout [T, d] and g_aux = dL/daux.
 *
 * [KB "argmaxは離散なのに、Routerはなぜ学習できるのか"]: the chosen expert id
 * is discrete and gives no gradient; the output keeps the continuous gate
 * p_{i*}(x), through which the gradient reaches the softmax and W_r.  The
 * capacity cut is piecewise constant as well.  [LP 3.3]: f_i is discrete and
 * P_i continuous, so the loss reaches the router through P_i only.  The rest
 * is the chain rule on the forward's definition:
 *   kept t (expert e, gate g):  u = W_in[e] x, a = relu(u), E = W_out[e] a,
 *     dE = g G_t, dg_t = G_t . E, du = (W_out[e]^T dE) * [u > 0],
 *     dW_out[e] += dE a^T,  dW_in[e] += du x_t^T,  dx_t += W_in[e]^T du;
 *   every t:  p = softmax(h_t),
 *     dp_i = [i = e_t and kept] dg_t + g_aux alpha N f_i / T   (f_i = load_i / T),
 *     dh = p * (dp - p . dp),  dW_r += dh x_t^T,  db += dh,  dx_t += W_r^T dh,
 *     dx_t += G_t (the residual).
 * The routing (expert_idx, gate, drop), the logits h and load are the
 * forward's.  Sums over tokens run in token order; OpenMP splits tokens or
 * experts.  db may be NULL.
 * ------------------------------------------------------------------------ */
void oracle_backward(const float* x, const float* W_r, const float* W_in, const float* W_out,
                     const double* h, const int32_t* expert_idx, const double* gate,
                     const uint8_t* drop, const int32_t* load, const double* G, double g_aux,
                     double alpha, int64_t T, int64_t d, int64_t F, int64_t N, double* dx,
                     double* dW_r, double* db, double* dW_in, double* dW_out, int nthreads) {
  double* dg = (double*)calloc((size_t)(T > 0 ? T : 1), sizeof(double));
  double* dh = (double*)calloc((size_t)(T > 0 ? T : 1) * (size_t)N, sizeof(double));

  /* expert path of dx and dg, per token */
#pragma omp parallel for schedule(dynamic, 4) num_threads(NT(nthreads))
  for (int64_t t = 0; t < T; ++t) {
    const float* xt = x + t * d;
    const double* Gt = G + t * d;
    for (int64_t k = 0; k < d; ++k) dx[t * d + k] = Gt[k];
    if (drop[t]) continue;
    const int64_t e = expert_idx[t];
    const float* Wi = W_in + e * F * d;
    const float* Wo = W_out + e * d * F;
    double* u = (double*)malloc(sizeof(double) * (size_t)F);
    double* du = (double*)malloc(sizeof(double) * (size_t)F);
    for (int64_t j = 0; j < F; ++j) {
      double acc = 0.0;
      for (int64_t k = 0; k < d; ++k) acc += (double)Wi[j * d + k] * (double)xt[k];
      u[j] = acc;
    }
    double s = 0.0;  /* dg = G . E, E_i = sum_j Wo[i, j] relu(u_j) */
    for (int64_t i = 0; i < d; ++i) {
      double E = 0.0;
      for (int64_t j = 0; j < F; ++j) E += (double)Wo[i * F + j] * (u[j] > 0.0 ? u[j] : 0.0);
      s += Gt[i] * E;
    }
    dg[t] = s;
    for (int64_t j = 0; j < F; ++j) {
      double acc = 0.0;
      if (u[j] > 0.0)
        for (int64_t i = 0; i < d; ++i) acc += (double)Wo[i * F + j] * gate[t] * Gt[i];
      du[j] = acc;
    }
    for (int64_t k = 0; k < d; ++k) {
      double acc = 0.0;
      for (int64_t j = 0; j < F; ++j) acc += (double)Wi[j * d + k] * du[j];
      dx[t * d + k] += acc;
    }
    free(u);
    free(du);
  }

  /* router path: softmax Jacobian on each token's logits */
#pragma omp parallel for schedule(static) num_threads(NT(nthreads))
  for (int64_t t = 0; t < T; ++t) {
    const double* ht = h + t * N;
    double m = ht[0];
    for (int64_t i = 1; i < N; ++i) m = ht[i] > m ? ht[i] : m;
    double S = 0.0;
    for (int64_t i = 0; i < N; ++i) S += exp(ht[i] - m);
    double pdp = 0.0;
    for (int64_t i = 0; i < N; ++i) {
      const double p = exp(ht[i] - m) / S;
      double dp = g_aux * alpha * (double)N * ((double)load[i] / (double)T) / (double)T;
      if (i == expert_idx[t] && !drop[t]) dp += dg[t];
      dh[t * N + i] = dp;       /* dp for now */
      pdp += p * dp;
    }
    for (int64_t i = 0; i < N; ++i) {
      const double p = exp(ht[i] - m) / S;
      dh[t * N + i] = p * (dh[t * N + i] - pdp);
    }
    for (int64_t k = 0; k < d; ++k) {
      double acc = 0.0;
      for (int64_t i = 0; i < N; ++i) acc += (double)W_r[i * d + k] * dh[t * N + i];
      dx[t * d + k] += acc;
    }
  }

  /* router weight and bias gradients: sums over tokens, per expert row */
#pragma omp parallel for schedule(static) num_threads(NT(nthreads))
  for (int64_t i = 0; i < N; ++i) {
    double bsum = 0.0;
    for (int64_t k = 0; k < d; ++k) dW_r[i * d + k] = 0.0;
    for (int64_t t = 0; t < T; ++t) {
      const double v = dh[t * N + i];
      bsum += v;
      for (int64_t k = 0; k < d; ++k) dW_r[i * d + k] += v * (double)x[t * d + k];
    }
    if (db) db[i] = bsum;
  }

  /* expert weight gradients: per expert, its kept tokens in token order */
#pragma omp parallel for schedule(dynamic, 1) num_threads(NT(nthreads))
  for (int64_t e = 0; e < N; ++e) {
    const float* Wi = W_in + e * F * d;
    const float* Wo = W_out + e * d * F;
    double* gWi = dW_in + e * F * d;
    double* gWo = dW_out + e * d * F;
    for (int64_t q = 0; q < F * d; ++q) gWi[q] = 0.0;
    for (int64_t q = 0; q < d * F; ++q) gWo[q] = 0.0;
    double* u = (double*)malloc(sizeof(double) * (size_t)F);
    double* du = (double*)malloc(sizeof(double) * (size_t)F);
    for (int64_t t = 0; t < T; ++t) {
      if (drop[t] || expert_idx[t] != e) continue;
      const float* xt = x + t * d;
      const double* Gt = G + t * d;
      for (int64_t j = 0; j < F; ++j) {
        double acc = 0.0;
        for (int64_t k = 0; k < d; ++k) acc += (double)Wi[j * d + k] * (double)xt[k];
        u[j] = acc;
      }
      for (int64_t j = 0; j < F; ++j) {
        double acc = 0.0;
        if (u[j] > 0.0)
          for (int64_t i = 0; i < d; ++i) acc += (double)Wo[i * F + j] * gate[t] * Gt[i];
        du[j] = acc;
      }
      for (int64_t i = 0; i < d; ++i) {
        const double dE = gate[t] * Gt[i];
        for (int64_t j = 0; j < F; ++j) gWo[i * F + j] += dE * (u[j] > 0.0 ? u[j] : 0.0);
      }
      for (int64_t j = 0; j < F; ++j)
        for (int64_t k = 0; k < d; ++k) gWi[j * d + k] += du[j] * (double)xt[k];
    }
    free(u);
    free(du);
  }
  free(dg);
  free(dh);
}

/* ------------------------------------------------------------------------
 * Backward pass of the top-k layer (the classic routing the Switch layer
 * reduces to k = 1; llm-papers-study section 3.1): the same chain rule with
 * every kept choice j of token t contributing its own gated expert output,
 *   out_t = x_t + sum_j [kept] g_tj E_{e_tj}(x_t),   g_tj = p_{e_tj}(h_t),
 * and with f_i = load_i / (k T) in the loss (load_i counts assignments), so
 *   dg_tj = G_t . E_{e_tj}(x_t),
 *   dp_i = sum_j [i = e_tj and kept] dg_tj + g_aux alpha N load_i / (k T^2),
 *   and each kept (t, j) adds its expert terms as in oracle_backward.
 * expert_idx, gate and drop are [T, k] in (token, choice) order.
 * ------------------------------------------------------------------------ */
void oracle_backward_topk(const float* x, const float* W_r, const float* W_in,
                          const float* W_out, const double* h, const int32_t* expert_idx,
                          const double* gate, const uint8_t* drop, const int32_t* load,
                          const double* G, double g_aux, double alpha, int64_t T, int64_t k,
                          int64_t d, int64_t F, int64_t N, double* dx, double* dW_r, double* db,
                          double* dW_in, double* dW_out, int nthreads) {
  double* dg = (double*)calloc((size_t)(T > 0 ? T * k : 1), sizeof(double));
  double* dh = (double*)calloc((size_t)(T > 0 ? T : 1) * (size_t)N, sizeof(double));

  /* expert path of dx and dg, per token and kept choice */
#pragma omp parallel for schedule(dynamic, 4) num_threads(NT(nthreads))
  for (int64_t t = 0; t < T; ++t) {
    const float* xt = x + t * d;
    const double* Gt = G + t * d;
    for (int64_t q = 0; q < d; ++q) dx[t * d + q] = Gt[q];
    double* u = (double*)malloc(sizeof(double) * (size_t)F);
    double* du = (double*)malloc(sizeof(double) * (size_t)F);
    for (int64_t j = 0; j < k; ++j) {
      const int64_t a = t * k + j;
      if (drop[a]) continue;
      const int64_t e = expert_idx[a];
      const float* Wi = W_in + e * F * d;
      const float* Wo = W_out + e * d * F;
      for (int64_t f = 0; f < F; ++f) {
        double acc = 0.0;
        for (int64_t q = 0; q < d; ++q) acc += (double)Wi[f * d + q] * (double)xt[q];
        u[f] = acc;
      }
      double s = 0.0;
      for (int64_t i = 0; i < d; ++i) {
        double E = 0.0;
        for (int64_t f = 0; f < F; ++f) E += (double)Wo[i * F + f] * (u[f] > 0.0 ? u[f] : 0.0);
        s += Gt[i] * E;
      }
      dg[a] = s;
      for (int64_t f = 0; f < F; ++f) {
        double acc = 0.0;
        if (u[f] > 0.0)
          for (int64_t i = 0; i < d; ++i) acc += (double)Wo[i * F + f] * gate[a] * Gt[i];
        du[f] = acc;
      }
      for (int64_t q = 0; q < d; ++q) {
        double acc = 0.0;
        for (int64_t f = 0; f < F; ++f) acc += (double)Wi[f * d + q] * du[f];
        dx[t * d + q] += acc;
      }
    }
    free(u);
    free(du);
  }

  /* router path: softmax Jacobian on each token's logits */
#pragma omp parallel for schedule(static) num_threads(NT(nthreads))
  for (int64_t t = 0; t < T; ++t) {
    const double* ht = h + t * N;
    double m = ht[0];
    for (int64_t i = 1; i < N; ++i) m = ht[i] > m ? ht[i] : m;
    double S = 0.0;
    for (int64_t i = 0; i < N; ++i) S += exp(ht[i] - m);
    double pdp = 0.0;
    for (int64_t i = 0; i < N; ++i) {
      const double p = exp(ht[i] - m) / S;
      double dp = g_aux * alpha * (double)N * ((double)load[i] / ((double)k * (double)T)) /
                  (double)T;
      for (int64_t j = 0; j < k; ++j)
        if (i == expert_idx[t * k + j] && !drop[t * k + j]) dp += dg[t * k + j];
      dh[t * N + i] = dp;
      pdp += p * dp;
    }
    for (int64_t i = 0; i < N; ++i) {
      const double p = exp(ht[i] - m) / S;
      dh[t * N + i] = p * (dh[t * N + i] - pdp);
    }
    for (int64_t q = 0; q < d; ++q) {
      double acc = 0.0;
      for (int64_t i = 0; i < N; ++i) acc += (double)W_r[i * d + q] * dh[t * N + i];
      dx[t * d + q] += acc;
    }
  }

  /* router weight and bias gradients: sums over tokens, per expert row */
#pragma omp parallel for schedule(static) num_threads(NT(nthreads))
  for (int64_t i = 0; i < N; ++i) {
    double bsum = 0.0;
    for (int64_t q = 0; q < d; ++q) dW_r[i * d + q] = 0.0;
    for (int64_t t = 0; t < T; ++t) {
      const double v = dh[t * N + i];
      bsum += v;
      for (int64_t q = 0; q < d; ++q) dW_r[i * d + q] += v * (double)x[t * d + q];
    }
    if (db) db[i] = bsum;
  }

  /* expert weight gradients: per expert, its kept assignments in (token, choice) order */
#pragma omp parallel for schedule(dynamic, 1) num_threads(NT(nthreads))
  for (int64_t e = 0; e < N; ++e) {
    const float* Wi = W_in + e * F * d;
    const float* Wo = W_out + e * d * F;
    double* gWi = dW_in + e * F * d;
    double* gWo = dW_out + e * d * F;
    for (int64_t q = 0; q < F * d; ++q) gWi[q] = 0.0;
    for (int64_t q = 0; q < d * F; ++q) gWo[q] = 0.0;
    double* u = (double*)malloc(sizeof(double) * (size_t)F);
    double* du = (double*)malloc(sizeof(double) * (size_t)F);
    for (int64_t a = 0; a < T * k; ++a) {
      if (drop[a] || expert_idx[a] != e) continue;
      const int64_t t = a / k;
      const float* xt = x + t * d;
      const double* Gt = G + t * d;
      for (int64_t f = 0; f < F; ++f) {
        double acc = 0.0;
        for (int64_t q = 0; q < d; ++q) acc += (double)Wi[f * d + q] * (double)xt[q];
        u[f] = acc;
      }
      for (int64_t f = 0; f < F; ++f) {
        double acc = 0.0;
        if (u[f] > 0.0)
          for (int64_t i = 0; i < d; ++i) acc += (double)Wo[i * F + f] * gate[a] * Gt[i];
        du[f] = acc;
      }
      for (int64_t i = 0; i < d; ++i) {
        const double dE = gate[a] * Gt[i];
        for (int64_t f = 0; f < F; ++f) gWo[i * F + f] += dE * (u[f] > 0.0 ? u[f] : 0.0);
      }
      for (int64_t f = 0; f < F; ++f)
        for (int64_t q = 0; q < d; ++q) gWi[f * d + q] += du[f] * (double)xt[q];
    }
    free(u);
    free(du);
  }
  free(dg);
  free(dh);
}
