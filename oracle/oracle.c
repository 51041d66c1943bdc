/*
 * oracle.c -- plain, slow fp64 CPU oracle for the Gemma 4 interleaved attention
 * block (sliding-window local attention and global attention with GQA, K=V and
 * p-RoPE).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file: only the tests, the smoke check of the package entry module and
 * the CPU-baseline leg of the benchmark use it.  It shares no code, header,
 * table or constant with the HIP library.
 *
 * What it computes is the plain definition of causal attention with rotary
 * position encoding, written out with no tiling, no online softmax, no
 * fusion: every output row is
 *     out[b,i,h] = sum_j w_j v_j / sum_j w_j,   w_j = exp(s_j - max_j s_j),
 *     s_j = <R(pos_i) q[b,i,h], R(pos_j) k[b,j,h/G]> / sqrt(d)
 * over the keys j that row i may see.  Sources, by page and section:
 *
 *  - Local vs global layers, window sizes, causal "whole preceding sequence":
 *    "Guia visual do Gemma 4" (pt.news.hada.io), section "Intercalacao de
 *    camadas de atencao (Interleaving Layers)"; and "Gemma 4: yak Google
 *    DeepMind ..." (techtoday.in.ua), section "Optymizovana uvaha: lokalni y
 *    hlobalni shary".
 *  - GQA (8 query heads per KV head in global layers; 2 in local layers):
 *    "Guia visual do Gemma 4", section "GQA (Grouped Query Attention)";
 *    techtoday page, same attention section.
 *  - K=V (keys and values are the same tensor in global layers):
 *    "Guia visual do Gemma 4", section "Tecnica K=V".
 *  - p-RoPE (only a fraction p of the rotary pairs is rotated; the
 *    low-frequency pairs are left alone to carry meaning):
 *    "Guia visual do Gemma 4", section "p-RoPE".
 *  - KV cache grows with prompt + generated tokens (decode):
 *    "Visao geral do modelo Gemma 4" (ai.google.dev), section "Principais
 *    Consideracoes para o planejamento de memoria".
 *
 * Readings taken where the pages are silent (each is listed with the others in
 * the design notes of the repository):
 *  - n_rot = floor(p * d / 2) pairs are rotated: pairs t = 0 .. n_rot-1, which
 *    are the highest-frequency ones; pair t occupies dims (2t, 2t+1) and turns
 *    by angle pos * theta^(-2t/d) (frequency over the full head dim d).
 *  - The rotation is counter-clockwise: (x, y) -> (x c - y s, x s + y c).
 *  - Window W keeps keys with 0 <= i - j < W (W keys including self); W = 0
 *    means unbounded (global).  Both layer kinds are causal.  The mask uses the
 *    sequence index; positions only feed the rotation.
 *  - Scores are scaled by 1/sqrt(d), d the layer's own head dim.
 *  - K=V: the same raw tensor is rotated for the scores and used raw as values.
 *  - Query head h reads KV head floor(h / G), G = Hq / Hkv.
 *
 * parity unpinned: the pair layout (adjacent pairs) and the frequency
 * convention are not fixed by any worked example on the pages; the pins in the
 * tests fix them only as the reading above.
 *
 * Inputs are read exactly (fp32, or bf16 bit patterns widened to fp64);
 * every intermediate is fp64; the softmax is two-pass.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define G4O_OK 0
#define G4O_EINVAL (-1)
#define G4O_ENOMEM (-2)

/* element idx of an input array of dtype 0 (fp32), 1 (bf16 bits) or 2 (fp64) */
static double g4o_in(const void* base, int dtype, size_t idx) {
  if (dtype == 0) return (double)((const float*)base)[idx];
  if (dtype == 2) return ((const double*)base)[idx];
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Number of rotated pairs for rotated fraction p of a head of dim d. */
int g4o_nrot(int d, double p) {
  int n = (int)floor(p * (double)d / 2.0);
  if (n < 0) n = 0;
  if (n > d / 2) n = d / 2;
  return n;
}

/* Angle of pair t at position pos: pos * theta^(-2t/d). */
static double g4o_angle(double pos, int t, int d, double theta) {
  return pos * pow(theta, -2.0 * (double)t / (double)d);
}

/* R(pos) applied in place to one head vector x[d] (p-RoPE section). */
void g4o_rope(double* x, int d, int n_rot, double theta, double pos) {
  for (int t = 0; t < n_rot; ++t) {
    double a = g4o_angle(pos, t, d, theta);
    double c = cos(a), s = sin(a);
    double x0 = x[2 * t], x1 = x[2 * t + 1];
    x[2 * t] = x0 * c - x1 * s;
    x[2 * t + 1] = x0 * s + x1 * c;
  }
}

/*
 * R(pos[i]) applied to every head vector of token i: x [n, H, d] of dtype 0
 * (fp32), 1 (bf16 bits) or 2 (fp64), pos [n]; out [n, H, d] fp64.  This is
 * the key a separate-key cache holds for token i (see g4o_decode).
 */
int g4o_rotate_rows(const void* x, int dtype, const int32_t* pos, int64_t n, int H, int d,
                    double theta, double p, double* out) {
  if (!x || !pos || !out || n < 0 || H <= 0 || d <= 0 || d % 2 || dtype < 0 || dtype > 2 ||
      !(theta > 0.0) || !(p >= 0.0 && p <= 1.0))
    return G4O_EINVAL;
  const int n_rot = g4o_nrot(d, p);
  for (int64_t i = 0; i < n; ++i)
    for (int h = 0; h < H; ++h) {
      const size_t off = ((size_t)i * H + h) * (size_t)d;
      for (int e = 0; e < d; ++e) out[off + e] = g4o_in(x, dtype, off + e);
      g4o_rope(out + off, d, n_rot, theta, (double)pos[i]);
    }
  return G4O_OK;
}

/* First visible key of query index i (window 0 = unbounded). */
static int64_t g4o_first_key(int64_t i, int window) {
  if (window <= 0) return 0;
  int64_t lo = i - window + 1;
  return lo < 0 ? 0 : lo;
}

static int g4o_check(int B, int S, int Hq, int Hkv, int d, int window, double theta, double p) {
  if (B < 0 || S < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || (d & 1)) return G4O_EINVAL;
  if (Hq % Hkv) return G4O_EINVAL;
  if (window < 0 || !(theta > 0.0) || !(p >= 0.0 && p <= 1.0)) return G4O_EINVAL;
  return G4O_OK;
}

/*
 * Causal prefill attention.
 *   q   [B, S, Hq,  d]     k, v [B, S, Hkv, d]   (k == v for the K=V layer)
 *   pos [B, S] int32 positions (rotation only)
 *   rows: NULL -> every row, out is [B, S, Hq, d];
 *         else nrows flattened row ids b*S + i, out is [nrows, Hq, d].
 * Returns 0, or a negative code for invalid arguments / out of memory.
 */
int g4o_prefill(const void* q, const void* k, const void* v, int dtype, const int32_t* pos,
                int B, int S, int Hq, int Hkv, int d, int window, double theta, double p,
                const int64_t* rows, int64_t nrows, double* out) {
  int rc = g4o_check(B, S, Hq, Hkv, d, window, theta, p);
  if (rc) return rc;
  if (!q || !k || !v || !pos || !out || (dtype != 0 && dtype != 1)) return G4O_EINVAL;
  const int G = Hq / Hkv;
  const int n_rot = g4o_nrot(d, p);
  const int64_t nr = rows ? nrows : (int64_t)B * S;
  if (nr == 0) return G4O_OK;
  for (int64_t r = 0; rows && r < nr; ++r)
    if (rows[r] < 0 || rows[r] >= (int64_t)B * S) return G4O_EINVAL;

  /* Cache of cos/sin of the key angles, per (b, j, pair): these depend only on
   * the key's position, so each is evaluated once. */
  const int64_t BS = (int64_t)B * S;
  double* cs = NULL;
  if (n_rot > 0) {
    cs = (double*)malloc(sizeof(double) * 2 * (size_t)BS * (size_t)n_rot);
    if (!cs) return G4O_ENOMEM;
    /* Only keys some requested row can see: per batch row b, the span from
     * the lowest first-visible key to the highest query index requested. */
    int64_t* lo = (int64_t*)malloc(sizeof(int64_t) * (size_t)B);
    int64_t* hi = (int64_t*)malloc(sizeof(int64_t) * (size_t)B);
    if (!lo || !hi) { free(cs); free(lo); free(hi); return G4O_ENOMEM; }
    for (int b = 0; b < B; ++b) { lo[b] = S; hi[b] = -1; }
    for (int64_t r = 0; r < nr; ++r) {
      int64_t row = rows ? rows[r] : r;
      int64_t b = row / S, i = row % S, j0 = g4o_first_key(i, window);
      if (j0 < lo[b]) lo[b] = j0;
      if (i > hi[b]) hi[b] = i;
    }
#pragma omp parallel for schedule(static)
    for (int64_t bj = 0; bj < BS; ++bj) {
      const int64_t b = bj / S, j = bj % S;
      if (j < lo[b] || j > hi[b]) continue;
      double P = (double)pos[bj];
      for (int t = 0; t < n_rot; ++t) {
        double a = g4o_angle(P, t, d, theta);
        cs[(bj * n_rot + t) * 2 + 0] = cos(a);
        cs[(bj * n_rot + t) * 2 + 1] = sin(a);
      }
    }
    free(lo);
    free(hi);
  }

  const double scale = 1.0 / sqrt((double)d);
  int err = 0;
#pragma omp parallel
  {
    double* qr = (double*)malloc(sizeof(double) * (size_t)G * d);
    double* kr = (double*)malloc(sizeof(double) * (size_t)d);
    double* sc = (double*)malloc(sizeof(double) * (size_t)G * (S > 0 ? S : 1));
    if (!qr || !kr || !sc) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t task = 0; task < nr * Hkv; ++task) {
        const int64_t r = task / Hkv;
        const int g = (int)(task % Hkv);
        const int64_t row = rows ? rows[r] : r;
        const int64_t b = row / S, i = row % S;
        const int64_t j0 = g4o_first_key(i, window);
        const int64_t nk = i - j0 + 1;
        /* rotated queries of the G heads that share KV head g */
        for (int hh = 0; hh < G; ++hh) {
          const int h = g * G + hh;
          const size_t qoff = (((size_t)b * S + i) * Hq + h) * (size_t)d;
          for (int e = 0; e < d; ++e) qr[hh * d + e] = g4o_in(q, dtype, qoff + e);
          g4o_rope(qr + hh * d, d, n_rot, theta, (double)pos[b * S + i]);
        }
        /* scores s_j for every visible key */
        for (int64_t jj = 0; jj < nk; ++jj) {
          const int64_t j = j0 + jj;
          const size_t koff = (((size_t)b * S + j) * Hkv + g) * (size_t)d;
          for (int e = 0; e < d; ++e) kr[e] = g4o_in(k, dtype, koff + e);
          const double* c = cs ? cs + ((size_t)(b * S + j) * n_rot) * 2 : NULL;
          for (int t = 0; t < n_rot; ++t) {
            double x0 = kr[2 * t], x1 = kr[2 * t + 1];
            kr[2 * t] = x0 * c[2 * t] - x1 * c[2 * t + 1];
            kr[2 * t + 1] = x0 * c[2 * t + 1] + x1 * c[2 * t];
          }
          for (int hh = 0; hh < G; ++hh) {
            double s = 0.0;
            for (int e = 0; e < d; ++e) s += qr[hh * d + e] * kr[e];
            sc[(size_t)hh * nk + jj] = s * scale;
          }
        }
        /* two-pass softmax and weighted sum of raw values */
        for (int hh = 0; hh < G; ++hh) {
          const int h = g * G + hh;
          double* o = out + ((size_t)r * Hq + h) * (size_t)d;
          double* srow = sc + (size_t)hh * nk;
          double m = -INFINITY;
          for (int64_t jj = 0; jj < nk; ++jj) if (srow[jj] > m) m = srow[jj];
          double l = 0.0;
          for (int64_t jj = 0; jj < nk; ++jj) { srow[jj] = exp(srow[jj] - m); l += srow[jj]; }
          for (int e = 0; e < d; ++e) o[e] = 0.0;
          for (int64_t jj = 0; jj < nk; ++jj) {
            const size_t voff = (((size_t)b * S + j0 + jj) * Hkv + g) * (size_t)d;
            const double w = srow[jj];
            for (int e = 0; e < d; ++e) o[e] += w * g4o_in(v, dtype, voff + e);
          }
          for (int e = 0; e < d; ++e) o[e] /= l;
        }
      }
    }
    free(qr); free(kr); free(sc);
  }
  free(cs);
  return err ? G4O_ENOMEM : G4O_OK;
}

/*
 * Probability row of query (b, i, h) over all S keys (0 outside the mask).
 * Debug output used by the tests: each row must sum to 1.
 */
int g4o_probs(const void* q, const void* k, int dtype, const int32_t* pos, int B, int S, int Hq,
              int Hkv, int d, int window, double theta, double p, int b, int i, int h,
              double* probs) {
  int rc = g4o_check(B, S, Hq, Hkv, d, window, theta, p);
  if (rc) return rc;
  if (!q || !k || !pos || !probs || b < 0 || b >= B || i < 0 || i >= S || h < 0 || h >= Hq)
    return G4O_EINVAL;
  const int G = Hq / Hkv, g = h / G, n_rot = g4o_nrot(d, p);
  double* qr = (double*)malloc(sizeof(double) * d);
  double* kr = (double*)malloc(sizeof(double) * d);
  if (!qr || !kr) { free(qr); free(kr); return G4O_ENOMEM; }
  const size_t qoff = (((size_t)b * S + i) * Hq + h) * (size_t)d;
  for (int e = 0; e < d; ++e) qr[e] = g4o_in(q, dtype, qoff + e);
  g4o_rope(qr, d, n_rot, theta, (double)pos[(size_t)b * S + i]);
  const int64_t j0 = g4o_first_key(i, window);
  double m = -INFINITY;
  for (int64_t j = 0; j < S; ++j) {
    if (j < j0 || j > i) { probs[j] = -INFINITY; continue; }
    const size_t koff = (((size_t)b * S + j) * Hkv + g) * (size_t)d;
    for (int e = 0; e < d; ++e) kr[e] = g4o_in(k, dtype, koff + e);
    g4o_rope(kr, d, n_rot, theta, (double)pos[(size_t)b * S + j]);
    double s = 0.0;
    for (int e = 0; e < d; ++e) s += qr[e] * kr[e];
    probs[j] = s / sqrt((double)d);
    if (probs[j] > m) m = probs[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < S; ++j) {
    probs[j] = (j < j0 || j > i) ? 0.0 : exp(probs[j] - m);
    l += probs[j];
  }
  for (int64_t j = 0; j < S; ++j) probs[j] /= l;
  free(qr); free(kr);
  return G4O_OK;
}

/*
 * Decode: one query token per sequence against a KV cache.
 *   q [B, Hq, d];  k_cache, v_cache [B, Hkv, capacity, d].
 *   With a value cache, k_cache holds every key already turned at its own
 *   position (R(t) k_t, as the fill writes it; values are never turned), so
 *   only the query is turned here.  v_cache NULL: K=V, k_cache holds the raw
 *   tensor, turned at each key's position for the scores and read raw as the
 *   values.
 *   pos [B]: position of the query token, whose own key is already cached.
 *   window > 0: ring cache, capacity == window, position t lives in slot
 *               t mod window; the query sees positions max(0, P-W+1) .. P.
 *   window = 0: linear cache, row t holds position t; the query sees 0 .. P.
 * A row whose position is negative, or beyond a linear cache, is all NaN.
 * This is row P of the prefill over the sequence the cache holds.
 */
int g4o_decode(const void* q, const void* kc, const void* vc, int dtype, const int32_t* pos, int B,
               int Hq, int Hkv, int d, int capacity, int window, double theta, double p,
               double* out) {
  int rc = g4o_check(B, 1, Hq, Hkv, d, window, theta, p);
  if (rc) return rc;
  if (!q || !kc || !pos || !out || capacity <= 0 || dtype < 0 || dtype > 2) return G4O_EINVAL;
  if (window > 0 && capacity != window) return G4O_EINVAL;
  const int key_turn = vc == NULL;  /* K=V: keys are turned here */
  if (!vc) vc = kc;
  const int G = Hq / Hkv, n_rot = g4o_nrot(d, p);
  const double scale = 1.0 / sqrt((double)d);
  int err = 0;
#pragma omp parallel
  {
    double* qr = (double*)malloc(sizeof(double) * (size_t)G * d);
    double* kr = (double*)malloc(sizeof(double) * d);
    double* sc = (double*)malloc(sizeof(double) * (size_t)G * (size_t)capacity);
    if (!qr || !kr || !sc) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t task = 0; task < (int64_t)B * Hkv; ++task) {
        const int b = (int)(task / Hkv), g = (int)(task % Hkv);
        const int64_t P = pos[b];
        const int bad = P < 0 || (window == 0 && P >= capacity);
        if (bad) {
          for (int hh = 0; hh < G; ++hh)
            for (int e = 0; e < d; ++e) out[((size_t)b * Hq + g * G + hh) * d + e] = NAN;
          continue;
        }
        const int64_t t0 = g4o_first_key(P, window);
        const int64_t nk = P - t0 + 1;
        for (int hh = 0; hh < G; ++hh) {
          const size_t qoff = ((size_t)b * Hq + g * G + hh) * (size_t)d;
          for (int e = 0; e < d; ++e) qr[hh * d + e] = g4o_in(q, dtype, qoff + e);
          g4o_rope(qr + hh * d, d, n_rot, theta, (double)P);
        }
        for (int64_t jj = 0; jj < nk; ++jj) {
          const int64_t t = t0 + jj;
          const int64_t slot = window > 0 ? t % window : t;
          const size_t koff = (((size_t)b * Hkv + g) * capacity + slot) * (size_t)d;
          for (int e = 0; e < d; ++e) kr[e] = g4o_in(kc, dtype, koff + e);
          if (key_turn) g4o_rope(kr, d, n_rot, theta, (double)t);
          for (int hh = 0; hh < G; ++hh) {
            double s = 0.0;
            for (int e = 0; e < d; ++e) s += qr[hh * d + e] * kr[e];
            sc[(size_t)hh * nk + jj] = s * scale;
          }
        }
        for (int hh = 0; hh < G; ++hh) {
          double* o = out + ((size_t)b * Hq + g * G + hh) * (size_t)d;
          double* srow = sc + (size_t)hh * nk;
          double m = -INFINITY;
          for (int64_t jj = 0; jj < nk; ++jj) if (srow[jj] > m) m = srow[jj];
          double l = 0.0;
          for (int64_t jj = 0; jj < nk; ++jj) { srow[jj] = exp(srow[jj] - m); l += srow[jj]; }
          for (int e = 0; e < d; ++e) o[e] = 0.0;
          for (int64_t jj = 0; jj < nk; ++jj) {
            const int64_t t = t0 + jj;
            const int64_t slot = window > 0 ? t % window : t;
            const size_t voff = (((size_t)b * Hkv + g) * capacity + slot) * (size_t)d;
            for (int e = 0; e < d; ++e) o[e] += srow[jj] * g4o_in(vc, dtype, voff + e);
          }
          for (int e = 0; e < d; ++e) o[e] /= l;
        }
      }
    }
    free(qr); free(kr); free(sc);
  }
  return err ? G4O_ENOMEM : G4O_OK;
}

/*
 * Cache fill: the k (and v) rows of a prefill, written into the decode
 * cache layout so that decoding continues where the prefill ended (the KV
 * cache grows with prompt and generated tokens: "Visao geral do modelo
 * Gemma 4", section "Principais Consideracoes para o planejamento de
 * memoria").
 *   k, v [B, S, Hkv, d] (v NULL: K=V, only k_cache is written), esize bytes
 *   per element (1 for fp8 codes already quantized by g4o_quantize_e4m3); pos [B, S]; k_cache, v_cache [B, Hkv, capacity, d].
 *   window > 0 (ring): the last min(S, capacity) tokens i of each sequence
 *     go to slot pos[b,i] mod capacity;
 *   window = 0 (linear): every token with 0 <= pos[b,i] < capacity goes to
 *     row pos[b,i].
 * Tokens with a negative position are not written.  Bytes are copied
 * unchanged; slots not written keep their contents.  The keys of a cache with
 * separate values are turned first (g4o_rotate_rows, then rounded to the
 * cache's element type); this function only places rows.
 */
int g4o_fill_cache(const void* k, const void* v, int esize, const int32_t* pos, int B, int S,
                   int Hkv, int d, int capacity, int window, void* k_cache, void* v_cache) {
  if (B < 0 || S < 0 || Hkv <= 0 || d <= 0 || capacity <= 0 || window < 0) return G4O_EINVAL;
  if ((esize != 1 && esize != 2 && esize != 4) || !k || !pos || !k_cache || (v && !v_cache))
    return G4O_EINVAL;
  const size_t row = (size_t)d * esize;
  for (int b = 0; b < B; ++b) {
    const int first = window > 0 && S > capacity ? S - capacity : 0;
    for (int i = first; i < S; ++i) {
      const int64_t P = pos[(size_t)b * S + i];
      if (P < 0 || (window == 0 && P >= capacity)) continue;
      const int64_t slot = window > 0 ? P % capacity : P;
      for (int g = 0; g < Hkv; ++g) {
        const size_t src = (((size_t)b * S + i) * Hkv + g) * row;
        const size_t dst = (((size_t)b * Hkv + g) * capacity + slot) * row;
        memcpy((char*)k_cache + dst, (const char*)k + src, row);
        if (v) memcpy((char*)v_cache + dst, (const char*)v + src, row);
      }
    }
  }
  return G4O_OK;
}

/*
 * Decode of L query tokens per sequence at once, the verify step of
 * speculative decoding (every model carries a draft model for it: "Visao
 * geral do modelo Gemma 4", section "Recursos"); L = 1 is ordinary decode.
 *   q [B, L, Hq, d]; k_cache, v_cache [B, Hkv, capacity, d] as for
 *   g4o_decode (with a value cache the keys are cached turned; v_cache NULL:
 *   K=V, raw); pos [B]: position P of the last query token.  Query
 *   token j sits at Pj = P - L + 1 + j, and the keys of all L tokens are
 *   already cached.
 *   window > 0: ring, position t in slot t mod capacity.  The ring holds
 *     positions P-capacity+1 .. P, so capacity >= window + L - 1 is required
 *     for the first query to find its whole window.  Query j sees positions
 *     max(0, Pj-window+1) .. Pj.
 *   window = 0: linear cache, row t holds position t; query j sees 0 .. Pj.
 * Rows of a query with Pj < 0, and every row of a sequence with P >= capacity
 * in a linear cache, are NaN.  Row j equals row Pj of the prefill over the
 * sequence the cache holds.
 */
int g4o_decode_multi(const void* q, const void* kc, const void* vc, int dtype, const int32_t* pos,
                     int B, int L, int Hq, int Hkv, int d, int capacity, int window, double theta,
                     double p, double* out) {
  int rc = g4o_check(B, 1, Hq, Hkv, d, window, theta, p);
  if (rc) return rc;
  if (!q || !kc || !pos || !out || capacity <= 0 || L < 1 || dtype < 0 || dtype > 2)
    return G4O_EINVAL;
  if (window > 0 && capacity < window + L - 1) return G4O_EINVAL;
  const int key_turn = vc == NULL;  /* K=V: keys are turned here */
  if (!vc) vc = kc;
  const int G = Hq / Hkv, n_rot = g4o_nrot(d, p);
  const double scale = 1.0 / sqrt((double)d);
  int err = 0;
#pragma omp parallel
  {
    double* qr = (double*)malloc(sizeof(double) * d);
    double* kr = (double*)malloc(sizeof(double) * d);
    double* sc = (double*)malloc(sizeof(double) * (size_t)capacity);
    if (!qr || !kr || !sc) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t task = 0; task < (int64_t)B * L * Hq; ++task) {
        const int b = (int)(task / ((int64_t)L * Hq));
        const int j = (int)(task / Hq % L), h = (int)(task % Hq), g = h / G;
        const int64_t P = pos[b], Pj = P - L + 1 + j;
        double* o = out + (((size_t)b * L + j) * Hq + h) * (size_t)d;
        if (P < 0 || Pj < 0 || (window == 0 && P >= capacity)) {
          for (int e = 0; e < d; ++e) o[e] = NAN;
          continue;
        }
        const int64_t t0 = g4o_first_key(Pj, window), nk = Pj - t0 + 1;
        const size_t qoff = (((size_t)b * L + j) * Hq + h) * (size_t)d;
        for (int e = 0; e < d; ++e) qr[e] = g4o_in(q, dtype, qoff + e);
        g4o_rope(qr, d, n_rot, theta, (double)Pj);
        for (int64_t jj = 0; jj < nk; ++jj) {
          const int64_t t = t0 + jj;
          const int64_t slot = window > 0 ? t % capacity : t;
          const size_t koff = (((size_t)b * Hkv + g) * capacity + slot) * (size_t)d;
          for (int e = 0; e < d; ++e) kr[e] = g4o_in(kc, dtype, koff + e);
          if (key_turn) g4o_rope(kr, d, n_rot, theta, (double)t);
          double s = 0.0;
          for (int e = 0; e < d; ++e) s += qr[e] * kr[e];
          sc[jj] = s * scale;
        }
        double m = -INFINITY;
        for (int64_t jj = 0; jj < nk; ++jj) if (sc[jj] > m) m = sc[jj];
        double l = 0.0;
        for (int64_t jj = 0; jj < nk; ++jj) { sc[jj] = exp(sc[jj] - m); l += sc[jj]; }
        for (int e = 0; e < d; ++e) o[e] = 0.0;
        for (int64_t jj = 0; jj < nk; ++jj) {
          const int64_t t = t0 + jj;
          const int64_t slot = window > 0 ? t % capacity : t;
          const size_t voff = (((size_t)b * Hkv + g) * capacity + slot) * (size_t)d;
          for (int e = 0; e < d; ++e) o[e] += sc[jj] * g4o_in(vc, dtype, voff + e);
        }
        for (int e = 0; e < d; ++e) o[e] /= l;
      }
    }
    free(qr); free(kr); free(sc);
  }
  return err ? G4O_ENOMEM : G4O_OK;
}

/*
 * Low-precision KV cache: FP8 E4M3 codes with a scale per KV head.
 *
 * The pages name optimized KV caches among the memory savings of the mobile
 * checkpoints and say the cache grows with every token ("Visao geral do modelo
 * Gemma 4", sections "Treinamento com reconhecimento de quantizacao (QAT)" and
 * "Principais Consideracoes para o planejamento de memoria"); they give no
 * format.  Reading taken: one byte per element in the OCP 8-bit floating-point
 * format E4M3 (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals at exponent 0, no infinities, S.1111.111 the only NaN), the
 * cached value being code value x scale[kv head].
 */

/* Value of E4M3 code c (0..255), from the format's definition. */
double g4o_e4m3_value(int c) {
  const int sign = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);          /* subnormal: m/8 * 2^(1-7) */
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);  /* normal: (1 + m/8) * 2^(e-7) */
  return sign ? -v : v;
}

/* E4M3 code of x: the nearest value of the format, a tie going to the one with
 * the even mantissa (round to nearest even); |x| at or beyond the largest value
 * 448 (infinities included) gives +-448; zero keeps its sign; NaN gives 0x7F. */
int g4o_e4m3_encode(float x) {
  if (isnan(x)) return 0x7F;
  const int sign = signbit(x) ? 0x80 : 0;
  double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E;
  if (a == 0.0) return sign;
  int e2;
  frexp(a, &e2);      /* a = f * 2^e2, f in [0.5, 1): a lies in binade [2^(e2-1), 2^e2) */
  int E = e2 - 1;
  if (E < -6) E = -6; /* below 2^-6 the subnormal spacing 2^-9 applies */
  /* the format has 8 values per binade: spacing 2^(E-3) */
  const double quantum = ldexp(1.0, E - 3);
  const double n = nearbyint(a / quantum); /* default rounding: ties to even */
  const double v = n * quantum;
  /* the code holding v (v <= 448 since a < 448 rounds to at most 448) */
  for (int c = 0; c < 0x7F; ++c)
    if (g4o_e4m3_value(c) == v) return sign | c;
  return -1;
}

/*
 * Quantize rows of a [rows, Hkv, d] tensor to E4M3 codes:
 *   out[r, h, e] = encode( fp32(x[r, h, e]) / scale[h] )
 * with the quotient rounded once to fp32 (IEEE division).  dtype: 0 fp32 or
 * 1 bf16 bits.
 */
int g4o_quantize_e4m3(const void* x, int dtype, const float* scale, int64_t rows, int Hkv, int d,
                      uint8_t* out) {
  if (!x || !scale || !out || rows < 0 || Hkv <= 0 || d <= 0 || (dtype != 0 && dtype != 1))
    return G4O_EINVAL;
  for (int64_t r = 0; r < rows; ++r)
    for (int h = 0; h < Hkv; ++h)
      for (int e = 0; e < d; ++e) {
        const size_t i = ((size_t)r * Hkv + h) * d + e;
        const float xf = (float)g4o_in(x, dtype, i); /* exact: the input is fp32 or bf16 */
        const float y = xf / scale[h];
        out[i] = (uint8_t)g4o_e4m3_encode(y);
      }
  return G4O_OK;
}

/*
 * Vision-encoder attention: 2D RoPE and no causal mask.
 *
 * Each patch carries a two-component grid position (w, h); head dims
 * [0, d/2) rotate by component w and [d/2, d) by component h ("Guia visual do
 * Gemma 4", sections "Encoder de visao" and "Suporte a proporcao variavel").
 * Readings taken where the page is silent:
 *  - the head dim d is split into halves [0, d/2) and [d/2, d); half c is an
 *    ordinary RoPE of a head of dim d/2 (pairs (2t, 2t+1) of the half, angle
 *    pos_c * theta^(-2t/(d/2)), counter-clockwise) driven by position
 *    component c, where component 0 is w and component 1 is h, the order the
 *    page names them;
 *  - every patch of an image attends to every patch of the image
 *    (bidirectional, as in a ViT: no causal mask, no window);
 *  - images in one batch may hold fewer than S patches: lengths[b] patches
 *    are valid, the keys past them are not attended to, and the output rows of
 *    the padding positions are zero.
 *   q [B,S,Hq,d], k, v [B,S,Hkv,d]; pos2 [B,S,2] int32 (w, h); lengths [B]
 *   int32 or NULL (all S); rows / nrows as for g4o_prefill.
 */
int g4o_vision_prefill(const void* q, const void* k, const void* v, int dtype,
                       const int32_t* pos2, const int32_t* lengths, int B, int S, int Hq, int Hkv,
                       int d, double theta, const int64_t* rows, int64_t nrows, double* out) {
  int rc = g4o_check(B, S, Hq, Hkv, d, 0, theta, 1.0);
  if (rc) return rc;
  if ((d % 4) || !q || !k || !v || !pos2 || !out || (dtype != 0 && dtype != 1)) return G4O_EINVAL;
  const int G = Hq / Hkv, half = d / 2;
  const double scale = 1.0 / sqrt((double)d);
  const int64_t n_out = rows ? nrows : (int64_t)B * S;
  int err = 0;
#pragma omp parallel
  {
    double* qr = (double*)malloc(sizeof(double) * d);
    double* kr = (double*)malloc(sizeof(double) * d);
    double* sc = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    if (!qr || !kr || !sc) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t task = 0; task < n_out * Hq; ++task) {
        const int64_t ri = task / Hq;
        const int h = (int)(task % Hq), g = h / G;
        const int64_t id = rows ? rows[ri] : ri;
        const int b = (int)(id / S), i = (int)(id % S);
        double* o = out + ((size_t)ri * Hq + h) * (size_t)d;
        int n = lengths ? lengths[b] : S;
        if (n < 0) n = 0;
        if (n > S) n = S;
        if (i >= n) {  /* padding patch */
          for (int e = 0; e < d; ++e) o[e] = 0.0;
          continue;
        }
        const size_t qoff = (((size_t)b * S + i) * Hq + h) * (size_t)d;
        const size_t pq = ((size_t)b * S + i) * 2;
        for (int e = 0; e < d; ++e) qr[e] = g4o_in(q, dtype, qoff + e);
        g4o_rope(qr, half, half / 2, theta, (double)pos2[pq]);
        g4o_rope(qr + half, half, half / 2, theta, (double)pos2[pq + 1]);
        for (int j = 0; j < n; ++j) {
          const size_t koff = (((size_t)b * S + j) * Hkv + g) * (size_t)d;
          const size_t pk = ((size_t)b * S + j) * 2;
          for (int e = 0; e < d; ++e) kr[e] = g4o_in(k, dtype, koff + e);
          g4o_rope(kr, half, half / 2, theta, (double)pos2[pk]);
          g4o_rope(kr + half, half, half / 2, theta, (double)pos2[pk + 1]);
          double s = 0.0;
          for (int e = 0; e < d; ++e) s += qr[e] * kr[e];
          sc[j] = s * scale;
        }
        double m = -INFINITY;
        for (int j = 0; j < n; ++j) if (sc[j] > m) m = sc[j];
        double l = 0.0;
        for (int j = 0; j < n; ++j) { sc[j] = exp(sc[j] - m); l += sc[j]; }
        for (int e = 0; e < d; ++e) o[e] = 0.0;
        for (int j = 0; j < n; ++j) {
          const size_t voff = (((size_t)b * S + j) * Hkv + g) * (size_t)d;
          for (int e = 0; e < d; ++e) o[e] += sc[j] * g4o_in(v, dtype, voff + e);
        }
        for (int e = 0; e < d; ++e) o[e] /= l;
      }
    }
    free(qr); free(kr); free(sc);
  }
  return err ? G4O_ENOMEM : G4O_OK;
}

/*
 * Threads of the OpenMP loops above: the count in use, and a setter so that a
 * caller can time the oracle on one thread as well as on all of them.  No
 * arithmetic.
 */
#include <omp.h>

int g4o_threads(void) { return omp_get_max_threads(); }

void g4o_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}
