/*
 * KDA oracle: the Kimi Delta Attention recurrence, token by token, in fp64.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. The GPU library neither links nor
 * includes anything from here, and this file includes nothing from it.
 *
 * What is computed, per sequence b and head h, for tokens t = 0 .. T-1:
 *
 *   1. Short causal convolution of width 4 on each raw projection channel
 *      (q, k and v), followed by SiLU. The three previous raw tokens come
 *      from a per-sequence ring (oldest first); the ring is session state.
 *      Source: "KV缓存从11.25GB缩到0.21GB：WARP中Kimi Delta Attention线性注意力
 *      原理剖析", section "KDA 递推公式先衰减再差分" (short conv, SiLU, 3-token
 *      ring) and the table under "414MB 的 KDA 状态从哪来" (3 projections).
 *   2. L2 normalisation of q and k over the head's d_k channels:
 *      x / sqrt(sum x^2 + eps). Same section ("q、k 在内核内部 L2 归一化").
 *      v is not normalised.
 *   3. Decay along the key axis: S'[i][j] = exp(g[i]) * S[i][j]; g is a
 *      log-space decay, exponentiated here. Same section, step (1).
 *   4. Delta read: r[j] = sum_i S'[i][j] * k[i].
 *   5. Rank-1 write: S[i][j] = S'[i][j] + beta * k[i] * (v[j] - r[j]).
 *      Same section, step (2); also "为什么 Kimi K3 敢把 KV Cache 扔掉？一篇讲透
 *      GPT-2 到 K3 的架构进化", section 7, the Kimi Linear update
 *      S_t = (I - beta k k^T) Diag(alpha) S_{t-1} + beta k v^T, which is the
 *      same algebra.
 *   6. Readout from the updated state: o[j] = sum_i S[i][j] * q[i].
 *      Section "KDA 递推公式先衰减再差分", step (3).
 *   7. Ring <- the last three raw tokens.
 *
 * Layouts (all row-major, fp64):
 *   q, k   [B][T][H][dk]      raw projections (or post-conv values, see flags)
 *   v      [B][T][H][dv]
 *   g      [B][T][H][dk]      natural-log decay per key channel
 *   beta   [B][T][H]
 *   conv_w [Ctot][4]          Ctot = H*(2*dk+dv); channels ordered q | k | v,
 *                             head-major inside each projection; tap 3
 *                             multiplies the current token, tap 0 the token
 *                             three steps back
 *   ring   [B][3][Ctot]       raw tokens t-3, t-2, t-1 (oldest first)
 *   S      [B][H][dk][dv]
 *   o      [B][T][H][dv]
 *
 * flags: 1 = inputs are already convolved and activated (steps 1 and 7 are
 * skipped, the ring is not touched); 2 = q and k are already normalised
 * (step 2 is skipped).
 *
 * Heads are independent, so (b, h) pairs run in parallel under OpenMP; each
 * pair is a plain sequential loop over tokens. No blocking, no reordering.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDAO_SKIP_CONV 1
#define KDAO_SKIP_L2 2

/* Number of threads the oracle will use (1 without OpenMP). */
int kdao_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static double silu(double y) { return y / (1.0 + exp(-y)); }

/* Step 1 for one channel c of sequence b at token t: the raw value of that
 * channel j steps back, taken from the inputs when it lies inside this call
 * and from the ring otherwise. */
static double raw_at(const double *x, long x_stride_t, int t, int back,
                     const double *ring_b, long Ctot, long c) {
  int s = t - back;
  if (s >= 0) return x[(long)s * x_stride_t];
  /* s = -1 is ring tap 2, s = -2 is tap 1, s = -3 is tap 0 */
  return ring_b[(long)(3 + s) * Ctot + c];
}

static double conv4_silu(const double *x, long x_stride_t, int t,
                         const double *ring_b, long Ctot, long c,
                         const double *w /* [4] for channel c */) {
  double y = w[0] * raw_at(x, x_stride_t, t, 3, ring_b, Ctot, c) +
             w[1] * raw_at(x, x_stride_t, t, 2, ring_b, Ctot, c) +
             w[2] * raw_at(x, x_stride_t, t, 1, ring_b, Ctot, c) +
             w[3] * raw_at(x, x_stride_t, t, 0, ring_b, Ctot, c);
  return silu(y);
}

static void l2_normalise(double *x, int n, double eps) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss + eps);
  for (int i = 0; i < n; ++i) x[i] *= inv;
}

/* Steps 1-2 for one (b, h) at token t: fills qh[dk], kh[dk], vh[dv]. */
static void prologue_token(int T, int H, int dk, int dv, int b, int h, int t,
                           const double *q, const double *k, const double *v,
                           const double *conv_w, const double *ring,
                           int flags, double eps,
                           double *qh, double *kh, double *vh) {
  const long Ctot = (long)H * (2 * dk + dv);
  const long sq_t = (long)H * dk, sv_t = (long)H * dv; /* token strides */
  const double *qb = q + ((long)b * T) * sq_t + (long)h * dk;
  const double *kb = k + ((long)b * T) * sq_t + (long)h * dk;
  const double *vb = v + ((long)b * T) * sv_t + (long)h * dv;
  const double *ring_b = ring ? ring + (long)b * 3 * Ctot : NULL;
  const long cq = (long)h * dk;                  /* channel of q[h][0] */
  const long ck = (long)H * dk + (long)h * dk;   /* channel of k[h][0] */
  const long cv = 2L * H * dk + (long)h * dv;    /* channel of v[h][0] */

  if (flags & KDAO_SKIP_CONV) {
    for (int i = 0; i < dk; ++i) qh[i] = qb[(long)t * sq_t + i];
    for (int i = 0; i < dk; ++i) kh[i] = kb[(long)t * sq_t + i];
    for (int j = 0; j < dv; ++j) vh[j] = vb[(long)t * sv_t + j];
  } else {
    for (int i = 0; i < dk; ++i)
      qh[i] = conv4_silu(qb + i, sq_t, t, ring_b, Ctot, cq + i,
                         conv_w + 4 * (cq + i));
    for (int i = 0; i < dk; ++i)
      kh[i] = conv4_silu(kb + i, sq_t, t, ring_b, Ctot, ck + i,
                         conv_w + 4 * (ck + i));
    for (int j = 0; j < dv; ++j)
      vh[j] = conv4_silu(vb + j, sv_t, t, ring_b, Ctot, cv + j,
                         conv_w + 4 * (cv + j));
  }
  if (!(flags & KDAO_SKIP_L2)) {
    l2_normalise(qh, dk, eps);
    l2_normalise(kh, dk, eps);
  }
}

/* Step 7 for the channels of head h of sequence b: ring <- last 3 raw tokens
 * of (old ring, x_0 .. x_{T-1}). */
static void ring_update(int T, int H, int dk, int dv, int b, int h,
                        const double *q, const double *k, const double *v,
                        double *ring) {
  const long Ctot = (long)H * (2 * dk + dv);
  double *ring_b = ring + (long)b * 3 * Ctot;
  const struct { const double *x; long stride_t; long c0; int n; } proj[3] = {
      {q + ((long)b * T) * H * dk + (long)h * dk, (long)H * dk, (long)h * dk, dk},
      {k + ((long)b * T) * H * dk + (long)h * dk, (long)H * dk,
       (long)H * dk + (long)h * dk, dk},
      {v + ((long)b * T) * H * dv + (long)h * dv, (long)H * dv,
       2L * H * dk + (long)h * dv, dv},
  };
  for (int p = 0; p < 3; ++p) {
    for (int i = 0; i < proj[p].n; ++i) {
      long c = proj[p].c0 + i;
      double nw[3];
      for (int tap = 0; tap < 3; ++tap) {
        /* new tap 0 holds x_{T-3}, tap 1 x_{T-2}, tap 2 x_{T-1} */
        int s = T - 3 + tap;
        nw[tap] = (s >= 0) ? proj[p].x[(long)s * proj[p].stride_t + i]
                           : ring_b[(long)(3 + s) * Ctot + c];
      }
      for (int tap = 0; tap < 3; ++tap) ring_b[(long)tap * Ctot + c] = nw[tap];
    }
  }
}

/* Full forward over T tokens: steps 1-7. S and ring are updated in place;
 * o receives every token's readout. Returns 0, or -1 on bad arguments. */
int kdao_forward(int B, int T, int H, int dk, int dv,
                 const double *q, const double *k, const double *v,
                 const double *g, const double *beta, const double *conv_w,
                 double *ring, double *S, double *o, int flags, double eps,
                 int nthreads) {
  if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  if (!(flags & KDAO_SKIP_CONV) && (!conv_w || !ring)) return -1;
  if (nthreads <= 0) nthreads = kdao_max_threads();
  const long BH = (long)B * H;
  int bad = 0;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (long bh = 0; bh < BH; ++bh) {
    const int b = (int)(bh / H), h = (int)(bh % H);
    double *qh = malloc(sizeof(double) * dk);
    double *kh = malloc(sizeof(double) * dk);
    double *vh = malloc(sizeof(double) * dv);
    double *r = malloc(sizeof(double) * dv);
    if (!qh || !kh || !vh || !r) {
#pragma omp atomic write
      bad = 1;
      free(qh); free(kh); free(vh); free(r);
      continue;
    }
    double *Sbh = S + bh * dk * dv;

    for (int t = 0; t < T; ++t) {
      prologue_token(T, H, dk, dv, b, h, t, q, k, v, conv_w, ring, flags, eps,
                     qh, kh, vh);
      const double *gt = g + (((long)b * T + t) * H + h) * dk;
      const double bt = beta[((long)b * T + t) * H + h];

      /* step 3: decay each key row i by exp(g[i]) */
      for (int i = 0; i < dk; ++i) {
        const double a = exp(gt[i]);
        for (int j = 0; j < dv; ++j) Sbh[(long)i * dv + j] *= a;
      }
      /* step 4: r = S'^T k */
      for (int j = 0; j < dv; ++j) r[j] = 0.0;
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) r[j] += Sbh[(long)i * dv + j] * kh[i];
      /* step 5: S = S' + beta k (v - r)^T */
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
          Sbh[(long)i * dv + j] += bt * kh[i] * (vh[j] - r[j]);
      /* step 6: o = S^T q */
      double *ot = o + (((long)b * T + t) * H + h) * dv;
      for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += Sbh[(long)i * dv + j] * qh[i];
        ot[j] = acc;
      }
    }
    /* step 7 */
    if (!(flags & KDAO_SKIP_CONV) && T > 0)
      ring_update(T, H, dk, dv, b, h, q, k, v, ring);
    free(qh); free(kh); free(vh); free(r);
  }
  return bad ? -1 : 0;
}

/* Steps 1, 2 and 7 only: the activations the recurrence consumes.
 * qo, ko [B][T][H][dk] and vo [B][T][H][dv] receive q-hat, k-hat (normalised
 * unless flags has bit 2) and v after conv and SiLU. The ring is advanced. */
int kdao_prologue(int B, int T, int H, int dk, int dv,
                  const double *q, const double *k, const double *v,
                  const double *conv_w, double *ring,
                  double *qo, double *ko, double *vo, int flags, double eps,
                  int nthreads) {
  if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  if (!(flags & KDAO_SKIP_CONV) && (!conv_w || !ring)) return -1;
  if (nthreads <= 0) nthreads = kdao_max_threads();
  const long BH = (long)B * H;

#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (long bh = 0; bh < BH; ++bh) {
    const int b = (int)(bh / H), h = (int)(bh % H);
    for (int t = 0; t < T; ++t) {
      double *qt = qo + (((long)b * T + t) * H + h) * dk;
      double *kt = ko + (((long)b * T + t) * H + h) * dk;
      double *vt = vo + (((long)b * T + t) * H + h) * dv;
      prologue_token(T, H, dk, dv, b, h, t, q, k, v, conv_w, ring, flags, eps,
                     qt, kt, vt);
    }
    if (!(flags & KDAO_SKIP_CONV) && T > 0)
      ring_update(T, H, dk, dv, b, h, q, k, v, ring);
  }
  return 0;
}

/* Output gate after the readout (a separate step, not part of the recurrence):
 * a gated RMSNorm of each head's readout vector. The C engine of "KV缓存从
 * 11.25GB缩到0.21GB：WARP中Kimi Delta Attention线性注意力原理剖析" lists a gated
 * RMSNorm beside the KDA decode step (section "相关源码与文档导航"), and "为什么
 * Kimi K3 敢把 KV Cache 扔掉？…" section 6 puts a gate on the output that
 * rescales features; neither prints the formula. The reading taken here: per row (one
 * token of one head) of n values x with gate pre-activations z,
 *
 *   y[j] = x[j] / sqrt(mean_j x[j]^2 + eps) * w[j] * sigmoid(z[j]),
 *
 * sigmoid(z) = 1 / (1 + exp(-z)), w a weight vector of length n shared by the
 * heads. x, z, y are [rows][n]; y may equal x. */
int kdao_gated_rmsnorm(long rows, int n, const double *x, const double *z,
                       const double *w, double eps, double *y) {
  if (rows < 0 || n <= 0 || !x || !z || !w || !y) return -1;
  for (long r = 0; r < rows; ++r) {
    const double *xr = x + r * n, *zr = z + r * n;
    double *yr = y + r * n;
    double ss = 0.0;
    for (int j = 0; j < n; ++j) ss += xr[j] * xr[j];
    const double rms = sqrt(ss / n + eps);
    for (int j = 0; j < n; ++j) {
      const double gate = 1.0 / (1.0 + exp(-zr[j]));
      yr[j] = xr[j] / rms * w[j] * gate;
    }
  }
  return 0;
}

/* Gates from raw projections (a separate step before the recurrence): the
 * Alpha/Beta projection of "为什么 Kimi K3 敢把 KV Cache 扔掉？…" section 6 sets
 * the forgetting strength alpha in [0, 1] and the update strength beta; the
 * squashing into (0, 1) by a logistic sigmoid is a reading (no formula is
 * printed). With alpha = sigmoid(a) the log-space decay the recurrence takes
 * is g = log(sigmoid(a)) = -log(1 + exp(-a)), and beta = sigmoid(b).
 * a, g: n_g values; b, beta: n_b values. */
int kdao_gates_from_raw(long n_g, const double *a, double *g, long n_b, const double *b,
                        double *beta) {
  if (n_g < 0 || n_b < 0 || (n_g && (!a || !g)) || (n_b && (!b || !beta))) return -1;
  for (long i = 0; i < n_g; ++i) {
    /* -log(1 + e^{-a}) written so that neither branch overflows */
    g[i] = a[i] >= 0.0 ? -log1p(exp(-a[i])) : a[i] - log1p(exp(a[i]));
  }
  for (long i = 0; i < n_b; ++i) beta[i] = 1.0 / (1.0 + exp(-b[i]));
  return 0;
}

/* Gradient of the recurrence (steps 3-6) for training: given the activations
 * q^, k^, v^ [B][T][H][d], g [B][T][H][dk], beta [B][T][H], the entering state
 * S0 [B][H][dk][dv] and the gradients dO [B][T][H][dv] of the readouts and
 * dST [B][H][dk][dv] of the final state, returns dq, dk [B][T][H][dk], dv
 * [B][T][H][dv], dg [B][T][H][dk], dbeta [B][T][H] and dS0 [B][H][dk][dv].
 *
 * Written from the update of section "KDA 递推公式先衰减再差分" by reverse-mode
 * differentiation, token by token from the last one. With S' = Diag(e^g) S_{t-1},
 * r = S'^T k, delta = beta (v - r), S_t = S' + k delta^T, o_t = S_t^T q and
 * G = dL/dS_t (the readouts of tokens t and later, and dST):
 *   G       += q do^T                  (o_t = S_t^T q)
 *   dq       = S_t do
 *   ddelta   = G^T k,  dk += G delta    (S_t = S' + k delta^T)
 *   dv       = beta ddelta,  dbeta = ddelta . (v - r),  dr = -beta ddelta
 *   dS'      = G + k dr^T,  dk += S' dr (r = S'^T k)
 *   dg[i]    = sum_j dS'[i][j] S'[i][j]
 *   G        = Diag(e^g) dS'           (dL/dS_{t-1})
 * and dS0 is the last G. The states S_t are kept from a forward pass, so this
 * is for small inputs only. Returns 0, or -1 on bad arguments. */
int kdao_core_backward(int B, int T, int H, int dk, int dv,
                       const double *q, const double *k, const double *v,
                       const double *g, const double *beta, const double *S0,
                       const double *dO, const double *dST,
                       double *dq, double *dk_out, double *dv_out, double *dg,
                       double *dbeta, double *dS0) {
  if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  const long BH = (long)B * H, SS = (long)dk * dv;
  double *states = malloc(sizeof(double) * SS * (T + 1));
  double *G = malloc(sizeof(double) * SS);
  double *Sp = malloc(sizeof(double) * SS);
  double *r = malloc(sizeof(double) * dv);
  double *del = malloc(sizeof(double) * dv);
  double *dd = malloc(sizeof(double) * dv);
  int bad = !states || !G || !Sp || !r || !del || !dd;
  for (long bh = 0; bh < BH && !bad; ++bh) {
    const int b = (int)(bh / H), h = (int)(bh % H);
#define TOK(t) (((long)b * T + (t)) * H + h)
    /* forward, keeping S_0 .. S_T */
    memcpy(states, S0 + bh * SS, sizeof(double) * SS);
    for (int t = 0; t < T; ++t) {
      const double *kt = k + TOK(t) * dk, *vt = v + TOK(t) * dv, *gt = g + TOK(t) * dk;
      const double bt = beta[TOK(t)];
      double *Sn = states + (long)(t + 1) * SS;
      const double *Sc = states + (long)t * SS;
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) Sn[(long)i * dv + j] = exp(gt[i]) * Sc[(long)i * dv + j];
      for (int j = 0; j < dv; ++j) {
        r[j] = 0.0;
        for (int i = 0; i < dk; ++i) r[j] += Sn[(long)i * dv + j] * kt[i];
      }
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) Sn[(long)i * dv + j] += bt * kt[i] * (vt[j] - r[j]);
    }
    /* backward */
    memcpy(G, dST + bh * SS, sizeof(double) * SS);
    for (int t = T - 1; t >= 0; --t) {
      const double *qt = q + TOK(t) * dk, *kt = k + TOK(t) * dk, *vt = v + TOK(t) * dv;
      const double *gt = g + TOK(t) * dk, *dot = dO + TOK(t) * dv;
      const double bt = beta[TOK(t)];
      const double *Sprev = states + (long)t * SS, *St = states + (long)(t + 1) * SS;
      double *dqt = dq + TOK(t) * dk, *dkt = dk_out + TOK(t) * dk, *dvt = dv_out + TOK(t) * dv;
      double *dgt = dg + TOK(t) * dk;
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) {
          G[(long)i * dv + j] += qt[i] * dot[j];
          Sp[(long)i * dv + j] = exp(gt[i]) * Sprev[(long)i * dv + j];
        }
      for (int j = 0; j < dv; ++j) {
        r[j] = 0.0;
        dd[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
          r[j] += Sp[(long)i * dv + j] * kt[i];
          dd[j] += G[(long)i * dv + j] * kt[i];
        }
        del[j] = bt * (vt[j] - r[j]);
      }
      double db = 0.0;
      for (int j = 0; j < dv; ++j) {
        dvt[j] = bt * dd[j];
        db += dd[j] * (vt[j] - r[j]);
      }
      dbeta[TOK(t)] = db;
      for (int i = 0; i < dk; ++i) {
        double aq = 0.0, ak = 0.0, ag = 0.0;
        for (int j = 0; j < dv; ++j) {
          const double drj = -bt * dd[j];
          aq += St[(long)i * dv + j] * dot[j];
          ak += G[(long)i * dv + j] * del[j] + Sp[(long)i * dv + j] * drj;
          const double dsp = G[(long)i * dv + j] + kt[i] * drj;
          ag += dsp * Sp[(long)i * dv + j];
          G[(long)i * dv + j] = exp(gt[i]) * dsp;
        }
        dqt[i] = aq;
        dkt[i] = ak;
        dgt[i] = ag;
      }
    }
    memcpy(dS0 + bh * SS, G, sizeof(double) * SS);
#undef TOK
  }
  free(states); free(G); free(Sp); free(r); free(del); free(dd);
  return bad ? -1 : 0;
}

/* Gradient of steps 1-2 (the width-4 causal conv, SiLU, and the L2
 * normalisation of q and k) for training: given the raw projections q, k
 * [B][T][H][dk], v [B][T][H][dv], the conv weights [Ctot][4], the ring read
 * as history (ring0 [B][3][Ctot], NULL for zeros) and the gradients dqh,
 * dkh [B][T][H][dk], dvh [B][T][H][dv] of the activations q^, k^, v^,
 * returns dq, dk, dv (raw projections), dconv_w [Ctot][4] and dring
 * [B][3][Ctot] (the history). The ring the forward writes (the last three
 * raw tokens) is not differentiated.
 *
 * Written from steps 1-2 by reverse-mode differentiation, per channel c with
 * x_s the raw value at token s (s < 0 from the ring), y_t = sum_j w[c][j]
 * x_{t-3+j}, z_t = SiLU(y_t) = y_t s(y_t), s the logistic sigmoid:
 *   q and k (per token and head, over d_k):
 *     u = |z|^2 + eps, q^ = z / sqrt(u),
 *     dz = (dq^ - q^ (q^ . dq^)) / sqrt(u);
 *   v: dz = dv^;
 *   dy = dz (s(y) + y s(y) (1 - s(y)));
 *   dx_{t-3+j} += w[c][j] dy_t,  dw[c][j] += dy_t x_{t-3+j}.
 * Returns 0, or -1 on bad arguments or allocation failure. */
int kdao_prologue_backward(int B, int T, int H, int dk, int dv,
                           const double *q, const double *k, const double *v,
                           const double *conv_w, const double *ring0,
                           const double *dqh, const double *dkh, const double *dvh,
                           double eps, double *dq, double *dk_out, double *dv_out,
                           double *dconv_w, double *dring) {
  if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
  const long Ctot = (long)H * (2 * dk + dv);
  const int nmax = dk > dv ? dk : dv;
  memset(dconv_w, 0, sizeof(double) * Ctot * 4);
  memset(dring, 0, sizeof(double) * (long)B * 3 * Ctot);
  double *xe = malloc(sizeof(double) * (long)(T + 3) * nmax);  /* [i][s + 3] */
  double *dxe = malloc(sizeof(double) * (long)(T + 3) * nmax);
  double *y = malloc(sizeof(double) * ((long)T * nmax + 1));     /* [t][i] */
  double *dz = malloc(sizeof(double) * ((long)T * nmax + 1));
  int bad = !xe || !dxe || !y || !dz;
  for (int b = 0; b < B && !bad; ++b)
    for (int h = 0; h < H; ++h)
      for (int p = 0; p < 3; ++p) {
        const int n = p < 2 ? dk : dv;
        const long st = (long)H * n;  /* token stride */
        const long c0 = p == 0 ? (long)h * dk : p == 1 ? (long)H * dk + (long)h * dk
                                                       : 2L * H * dk + (long)h * dv;
        const long base = (long)b * T * st + (long)h * n;
        const double *x = (p == 0 ? q : p == 1 ? k : v) + base;
        const double *dxh = (p == 0 ? dqh : p == 1 ? dkh : dvh) + base;
        double *dxo = (p == 0 ? dq : p == 1 ? dk_out : dv_out) + base;
        for (int i = 0; i < n; ++i)
          for (int s = -3; s < T; ++s) {
            double val = 0.0;
            if (s >= 0) val = x[(long)s * st + i];
            else if (ring0) val = ring0[((long)b * 3 + (3 + s)) * Ctot + c0 + i];
            xe[(long)i * (T + 3) + s + 3] = val;
            dxe[(long)i * (T + 3) + s + 3] = 0.0;
          }
        for (int t = 0; t < T; ++t) {
          double *yt = y + (long)t * n, *dzt = dz + (long)t * n;
          for (int i = 0; i < n; ++i) {
            const double *w = conv_w + 4 * (c0 + i);
            const double *xi = xe + (long)i * (T + 3) + t;  /* xi[j] = x_{t-3+j} */
            yt[i] = w[0] * xi[0] + w[1] * xi[1] + w[2] * xi[2] + w[3] * xi[3];
          }
          if (p < 2) {
            double ss = 0.0;
            for (int i = 0; i < n; ++i) {
              const double zi = silu(yt[i]);
              ss += zi * zi;
            }
            const double nrm = sqrt(ss + eps);
            double dot = 0.0;
            for (int i = 0; i < n; ++i) dot += silu(yt[i]) / nrm * dxh[(long)t * st + i];
            for (int i = 0; i < n; ++i)
              dzt[i] = (dxh[(long)t * st + i] - silu(yt[i]) / nrm * dot) / nrm;
          } else {
            for (int i = 0; i < n; ++i) dzt[i] = dxh[(long)t * st + i];
          }
          for (int i = 0; i < n; ++i) {
            const double sg = 1.0 / (1.0 + exp(-yt[i]));
            const double dy = dzt[i] * (sg + yt[i] * sg * (1.0 - sg));
            const double *w = conv_w + 4 * (c0 + i);
            double *dw = dconv_w + 4 * (c0 + i);
            for (int j = 0; j < 4; ++j) {
              dxe[(long)i * (T + 3) + t + j] += w[j] * dy;
              dw[j] += dy * xe[(long)i * (T + 3) + t + j];
            }
          }
        }
        for (int i = 0; i < n; ++i) {
          for (int t = 0; t < T; ++t) dxo[(long)t * st + i] = dxe[(long)i * (T + 3) + t + 3];
          for (int s = 0; s < 3; ++s)
            dring[((long)b * 3 + s) * Ctot + c0 + i] = dxe[(long)i * (T + 3) + s];
        }
      }
  free(xe); free(dxe); free(y); free(dz);
  return bad ? -1 : 0;
}
