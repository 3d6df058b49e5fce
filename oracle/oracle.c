/*
 * oracle.c -- fp64 CPU oracle for batch-1 decode of a Llama decoder stack
 * whose projections are block-quantized (Q8_0, Q4_0, Q4_K, Q6_K).
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this file.  It shares no code, header or
 * table with the HIP library; it is the plain definition of what the decode
 * computes, in double precision, with sums taken in index order.
 *
 * What is computed, and where the pages state it (ntransformer pages; p1 is
 * the unwiki summary, p2 the GeekNews article):
 *   - weights stored in the GGUF formats Q8_0, Q4_0, Q4_K, Q5_K, Q6_K, F16
 *     and F32 (p1 "About" format list; p2 "Présentation de NTransformer");
 *   - the Llama decoder: RMSNorm, RoPE, grouped-query attention over a KV
 *     cache, SwiGLU FFN (p1 list of Llama features; p2 "Fonctionnalités
 *     principales", last bullet);
 *   - an F16 KV cache (p1 roadmap, phase 3; p2 "Feuille de route");
 *   - GEMV, RMSNorm, RoPE, SwiGLU and softmax as the per-token kernels, and a
 *     sampler (p2 "Architecture et structure du code");
 *   - self-speculative decoding, whose verify pass runs M drafted tokens
 *     through the stack (p1 feature list; p2 "Fonctionnalités principales");
 *     greedy speculative decoding emits exactly the plain greedy tokens, so
 *     the plain greedy stack is its oracle;
 *   - layer skip, the layers chosen by the cosine similarity of their input
 *     and output (p1 feature list and roadmap phase 3).
 * The pages stop at list level.  Where they are silent the oracle takes one
 * plain reading, marked READING below; the byte layouts of the K-quant
 * superblocks are the GGUF ones (READING: no format file is at hand, so the
 * compatibility of those two layouts with real GGUF files is parity
 * unpinned).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_Q8_0 = 0, OR_Q4_0 = 1, OR_Q4_K = 2, OR_Q6_K = 3, OR_Q5_K = 4, OR_F16 = 5, OR_F32 = 6 };

/* ---------------------------------------------------------------- scalars */

/* IEEE binary16 bits -> double (exact). */
double or_half(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(m + 1024), e - 25);
  return s ? -v : v;
}

/* double -> binary16 bits, round to nearest, ties to even (the rounding of
 * values appended to the F16 KV cache). */
uint16_t or_to_half(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (isnan(v)) return 0x7e00u;
  /* largest finite half is 65504; 65520 is the midpoint to 2^16 */
  if (a >= 65520.0) return sign | 0x7c00u;
  /* express a as an integer count of the half-precision unit at a's binade */
  int e = (a < 0x1p-14) ? -14 : ilogb(a);   /* exponent of the binade      */
  double unit = ldexp(1.0, e - 10);          /* spacing of halfs there      */
  double n = a / unit;                       /* exact: power-of-two scaling */
  double r = floor(n);
  double frac = n - r;
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  double q = r * unit;                       /* rounded magnitude           */
  if (q >= 65520.0) return sign | 0x7c00u;
  if (q < 0x1p-14) return sign | (uint16_t)(q / 0x1p-24);
  int E = ilogb(q);
  int mant = (int)(q / ldexp(1.0, E - 10)) - 1024;
  return sign | (uint16_t)((E + 15) << 10) | (uint16_t)mant;
}

int or_block_elems(int fmt) {
  switch (fmt) {
    case OR_Q8_0: case OR_Q4_0: return 32;
    case OR_Q4_K: case OR_Q6_K: case OR_Q5_K: return 256;
    case OR_F16: case OR_F32: return 1;    /* unquantized: one value per "block" */
  }
  return 0;
}

int or_block_bytes(int fmt) {
  switch (fmt) {
    case OR_Q8_0: return 2 + 32;            /* d, 32 x int8                 */
    case OR_Q4_0: return 2 + 16;            /* d, 32 nibbles                */
    case OR_Q4_K: return 2 + 2 + 12 + 128;  /* d, dmin, scales, 256 nibbles */
    case OR_Q6_K: return 128 + 64 + 16 + 2; /* ql, qh, scales, d            */
    case OR_Q5_K: return 2 + 2 + 12 + 32 + 128; /* d, dmin, scales, qh, nibbles */
    case OR_F16: return 2;
    case OR_F32: return 4;
  }
  return 0;
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ------------------------------------------------------------ block decode */

/* Q4_K: sub-block s (elements 32s..32s+31) has a 6-bit scale and a 6-bit
 * min.  READING (GGUF packing): for s < 4 they are the low six bits of bytes
 * s and s+4; for s >= 4 the low four bits come from byte s+4 (scale: low
 * nibble, min: high nibble) and the top two bits from the top two bits of
 * byte s-4 (scale) and byte s (min). */
static void q4k_scale_min(const uint8_t* sc, int s, int* scale, int* min) {
  if (s < 4) {
    *scale = sc[s] & 63;
    *min = sc[s + 4] & 63;
  } else {
    *scale = (sc[s + 4] & 15) | ((sc[s - 4] >> 6) << 4);
    *min = (sc[s + 4] >> 4) | ((sc[s] >> 6) << 4);
  }
}

/* Decode one block into its or_block_elems(fmt) weights, in element order. */
void or_dequant_block(int fmt, const uint8_t* b, double* w) {
  switch (fmt) {
    case OR_Q8_0: { /* w_j = d * q_j */
      double d = or_half(rd16(b));
      for (int j = 0; j < 32; ++j) w[j] = d * (double)(int8_t)b[2 + j];
      break;
    }
    case OR_Q4_0: { /* byte j: low nibble -> element j, high -> j+16; w = d (q - 8) */
      double d = or_half(rd16(b));
      const uint8_t* qs = b + 2;
      for (int j = 0; j < 16; ++j) {
        w[j] = d * (double)((qs[j] & 15) - 8);
        w[j + 16] = d * (double)((qs[j] >> 4) - 8);
      }
      break;
    }
    case OR_Q4_K: { /* w = d * scale_s * q - dmin * min_s */
      double d = or_half(rd16(b)), dmin = or_half(rd16(b + 2));
      const uint8_t* sc = b + 4;
      const uint8_t* qs = b + 16;
      for (int e = 0; e < 256; ++e) {
        int s = e / 32, scale, min;
        q4k_scale_min(sc, s, &scale, &min);
        /* READING (GGUF order): 64-element chunk c = e/64 uses bytes
         * 32c..32c+31; the first 32 elements of the chunk are the low
         * nibbles, the next 32 the high nibbles. */
        int c = e / 64, l = e % 32;
        uint8_t byte = qs[32 * c + l];
        int q = ((e / 32) % 2) ? (byte >> 4) : (byte & 15);
        w[e] = d * (double)scale * (double)q - dmin * (double)min;
      }
      break;
    }
    case OR_Q5_K: { /* w = d * scale_s * q - dmin * min_s, q 5-bit */
      double d = or_half(rd16(b)), dmin = or_half(rd16(b + 2));
      const uint8_t* sc = b + 4;
      const uint8_t* qh = b + 16;
      const uint8_t* qs = b + 48;
      for (int e = 0; e < 256; ++e) {
        /* READING (GGUF order; the pages only name the format): scales and
         * mins as Q4_K, the low four bits as Q4_K's nibbles, and the fifth
         * bit of element l (< 32) of sub-block s is bit s of qh[l]. */
        int s = e / 32, c = e / 64, l = e % 32, scale, min;
        q4k_scale_min(sc, s, &scale, &min);
        uint8_t byte = qs[32 * c + l];
        int q = ((s % 2) ? (byte >> 4) : (byte & 15)) | (((qh[l] >> s) & 1) << 4);
        w[e] = d * (double)scale * (double)q - dmin * (double)min;
      }
      break;
    }
    case OR_F16:
      w[0] = or_half(rd16(b));
      break;
    case OR_F32: { /* IEEE binary32, little endian */
      float f;
      memcpy(&f, b, 4);
      w[0] = (double)f;
      break;
    }
    case OR_Q6_K: { /* w_e = d * scale[e/16] * (q_e - 32) */
      const uint8_t* ql = b;
      const uint8_t* qh = b + 128;
      const int8_t* sc = (const int8_t*)(b + 192);
      double d = or_half(rd16(b + 208));
      for (int e = 0; e < 256; ++e) {
        /* READING (GGUF order): half n = e/128; within it, quarter k = (e%128)/32
         * and lane l = e%32.  Low four bits: nibble k/2 of ql[64n + 32(k%2) + l];
         * high two bits: bits 2k..2k+1 of qh[32n + l]. */
        int n = e / 128, k = (e % 128) / 32, l = e % 32;
        uint8_t lo = ql[64 * n + 32 * (k % 2) + l];
        int nib = (k / 2) ? (lo >> 4) : (lo & 15);
        int hi = (qh[32 * n + l] >> (2 * k)) & 3;
        int q = nib | (hi << 4);
        w[e] = d * (double)sc[e / 16] * (double)(q - 32);
      }
      break;
    }
  }
}

/* Decode `cols` weights of one row (row bytes laid out as consecutive blocks). */
void or_dequant_row(int fmt, const uint8_t* row, int64_t cols, double* w) {
  int qk = or_block_elems(fmt), bb = or_block_bytes(fmt);
  for (int64_t j = 0; j < cols / qk; ++j) or_dequant_block(fmt, row + j * bb, w + j * qk);
}

/* ------------------------------------------------------------------ GEMV */

/* y[r] = sum_k w[r][k] x[k], summed in k order (p2 "Architecture et structure
 * du code": GEMV over quantized weights).  Rows are independent; they are
 * spread over threads, each row's sum is sequential. */
void or_gemv(int fmt, const uint8_t* W, const double* x, double* y, int64_t rows, int64_t cols) {
  int qk = or_block_elems(fmt), bb = or_block_bytes(fmt);
  int64_t rb = cols / qk * bb;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double w[256];
    double acc = 0.0;
    const uint8_t* row = W + r * rb;
    for (int64_t j = 0; j < cols / qk; ++j) {
      or_dequant_block(fmt, row + j * bb, w);
      for (int e = 0; e < qk; ++e) acc += w[e] * x[j * qk + e];
    }
    y[r] = acc;
  }
}

/* Same, with an fp32 input vector widened exactly to double. */
void or_gemv_f32(int fmt, const uint8_t* W, const float* x32, double* y, int64_t rows, int64_t cols) {
  double* x = (double*)malloc(sizeof(double) * (size_t)cols);
  for (int64_t k = 0; k < cols; ++k) x[k] = (double)x32[k];
  or_gemv(fmt, W, x, y, rows, cols);
  free(x);
}

/* ------------------------------------------------------- layer components */

/* RMSNorm: out = x / sqrt(mean(x^2) + eps) * g.  READING: eps = 1e-5 is
 * passed in; the gain multiplies after normalisation. */
void or_rmsnorm(const double* x, const float* g, int64_t n, double eps, double* out) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
  double r = 1.0 / sqrt(ss / (double)n + eps);
  for (int64_t i = 0; i < n; ++i) out[i] = x[i] * r * (double)g[i];
}

/* RoPE at position pos over n_heads heads of head_dim values each.
 * READING: adjacent pairs (2i, 2i+1) of a head rotate by the angle
 * pos * theta^(-2i/head_dim); no frequency scaling. */
void or_rope(double* v, int n_heads, int head_dim, int64_t pos, double theta) {
  for (int h = 0; h < n_heads; ++h) {
    double* p = v + (int64_t)h * head_dim;
    for (int i = 0; i < head_dim / 2; ++i) {
      double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)head_dim);
      double c = cos(ang), s = sin(ang);
      double a = p[2 * i], b = p[2 * i + 1];
      p[2 * i] = a * c - b * s;
      p[2 * i + 1] = a * s + b * c;
    }
  }
}

/* Decode attention for one query token over cache positions 0..n_pos-1.
 * q: [n_head][hd]; caches: f16 [n_kv][max_ctx][hd]; o: [n_head][hd].
 * READING: query head h reads kv head h / (n_head / n_kv); scores are
 * q.k / sqrt(hd); softmax taken with the maximum subtracted. */
void or_attention(const double* q, const uint16_t* kc, const uint16_t* vc, int n_head, int n_kv,
                  int hd, int64_t max_ctx, int64_t n_pos, double* o) {
  int group = n_head / n_kv;
  double* s = (double*)malloc(sizeof(double) * (size_t)(n_pos > 0 ? n_pos : 1));
  for (int h = 0; h < n_head; ++h) {
    int g = h / group;
    const double* qh = q + (int64_t)h * hd;
    double m = -INFINITY;
    for (int64_t t = 0; t < n_pos; ++t) {
      const uint16_t* kr = kc + ((int64_t)g * max_ctx + t) * hd;
      double dot = 0.0;
      for (int d = 0; d < hd; ++d) dot += qh[d] * or_half(kr[d]);
      s[t] = dot / sqrt((double)hd);
      if (s[t] > m) m = s[t];
    }
    double z = 0.0;
    for (int64_t t = 0; t < n_pos; ++t) {
      s[t] = exp(s[t] - m);
      z += s[t];
    }
    double* oh = o + (int64_t)h * hd;
    for (int d = 0; d < hd; ++d) oh[d] = 0.0;
    for (int64_t t = 0; t < n_pos; ++t) {
      const uint16_t* vr = vc + ((int64_t)g * max_ctx + t) * hd;
      double p = s[t] / z;
      for (int d = 0; d < hd; ++d) oh[d] += p * or_half(vr[d]);
    }
  }
  free(s);
}

/* silu(z) = z / (1 + e^-z); for very negative z, e^-z overflows and the
 * quotient is -0, as IEEE arithmetic gives. */
double or_silu(double z) { return z / (1.0 + exp(-z)); }

/* ------------------------------------------------------------------ layer */

typedef struct {
  int32_t hidden, n_head, n_kv_head, head_dim, ffn;
  int64_t max_ctx;
  double rope_theta, rms_eps;
} or_cfg;

typedef struct {
  int32_t fmt;
  const uint8_t* data;
} or_mat;

typedef struct {
  const float *attn_norm, *ffn_norm;
  or_mat wq, wk, wv, wo, wg, wu, wd;
  uint16_t *k_cache, *v_cache; /* f16 [n_kv][max_ctx][head_dim] */
} or_layer_w;

/* One pre-norm Llama decoder layer over M tokens at positions pos..pos+M-1;
 * x is [M][hidden], updated in place.
 *   xn = RMSNorm(x, g_attn); q,k,v = Wq xn, Wk xn, Wv xn; RoPE(q, k);
 *   K,V[pos+i] = f16(k_i, v_i)  (round to nearest even);
 *   token i attends to positions 0..pos+i (the new entries read back as f16);
 *   h = x + Wo o; out = h + Wd (silu(Wg hn) * Wu hn), hn = RMSNorm(h, g_ffn).
 * READING: pre-norm with two residual adds; SwiGLU is silu(gate) * up. */
void or_layer(const or_cfg* c, const or_layer_w* L, double* x, int M, int64_t pos) {
  const int H = c->hidden, hd = c->head_dim;
  const int nq = c->n_head * hd, nkv = c->n_kv_head * hd;
  double* xn = (double*)malloc(sizeof(double) * H);
  double* q = (double*)malloc(sizeof(double) * (size_t)M * nq);
  double* k = (double*)malloc(sizeof(double) * nkv);
  double* v = (double*)malloc(sizeof(double) * nkv);
  double* o = (double*)malloc(sizeof(double) * nq);
  double* t = (double*)malloc(sizeof(double) * H);
  double* g = (double*)malloc(sizeof(double) * c->ffn);
  double* u = (double*)malloc(sizeof(double) * c->ffn);

  /* projections, RoPE and cache append for every new token first */
  for (int i = 0; i < M; ++i) {
    int64_t p = pos + i;
    or_rmsnorm(x + (int64_t)i * H, L->attn_norm, H, c->rms_eps, xn);
    or_gemv(L->wq.fmt, L->wq.data, xn, q + (int64_t)i * nq, nq, H);
    or_gemv(L->wk.fmt, L->wk.data, xn, k, nkv, H);
    or_gemv(L->wv.fmt, L->wv.data, xn, v, nkv, H);
    or_rope(q + (int64_t)i * nq, c->n_head, hd, p, c->rope_theta);
    or_rope(k, c->n_kv_head, hd, p, c->rope_theta);
    for (int kh = 0; kh < c->n_kv_head; ++kh)
      for (int d = 0; d < hd; ++d) {
        int64_t off = ((int64_t)kh * c->max_ctx + p) * hd + d;
        L->k_cache[off] = or_to_half(k[kh * hd + d]);
        L->v_cache[off] = or_to_half(v[kh * hd + d]);
      }
  }
  for (int i = 0; i < M; ++i) {
    double* xi = x + (int64_t)i * H;
    or_attention(q + (int64_t)i * nq, L->k_cache, L->v_cache, c->n_head, c->n_kv_head, hd, c->max_ctx,
                 pos + i + 1, o);
    or_gemv(L->wo.fmt, L->wo.data, o, t, H, nq);
    for (int r = 0; r < H; ++r) xi[r] += t[r]; /* h = x + Wo o */
    or_rmsnorm(xi, L->ffn_norm, H, c->rms_eps, xn);
    or_gemv(L->wg.fmt, L->wg.data, xn, g, c->ffn, H);
    or_gemv(L->wu.fmt, L->wu.data, xn, u, c->ffn, H);
    for (int r = 0; r < c->ffn; ++r) g[r] = or_silu(g[r]) * u[r];
    or_gemv(L->wd.fmt, L->wd.data, g, t, H, c->ffn);
    for (int r = 0; r < H; ++r) xi[r] += t[r]; /* out = h + Wd a */
  }
  free(xn); free(q); free(k); free(v); free(o); free(t); free(g); free(u);
}

/* Layer over an fp32 input [M][hidden]; the result is written in double. */
void or_layer_f32(const or_cfg* c, const or_layer_w* L, const float* x32, double* out, int M, int64_t pos) {
  for (int64_t i = 0; i < (int64_t)M * c->hidden; ++i) out[i] = (double)x32[i];
  or_layer(c, L, out, M, pos);
}

/* ------------------------------------------------------------------ stack */

typedef struct {
  or_cfg cfg;
  int32_t n_layer, vocab;
  or_mat tok_emb, lm_head; /* both [vocab][hidden] */
  const float* out_norm;
  const or_layer_w* layers;
} or_model;

/* Index of the largest value, lowest index among equal maxima; *margin gets
 * the gap to the runner-up (the largest value at any other index). */
int64_t or_argmax(const double* v, int64_t n, double* margin) {
  int64_t best = 0;
  for (int64_t i = 1; i < n; ++i)
    if (v[i] > v[best]) best = i;
  if (margin) {
    double second = -INFINITY;
    for (int64_t i = 0; i < n; ++i)
      if (i != best && v[i] > second) second = v[i];
    *margin = v[best] - second;
  }
  return best;
}

/* One decode (M = 1) or verify (M > 1) pass: embedding rows of tokens[0..M)
 * -> the layers at positions pos..pos+M-1 -> final RMSNorm -> LM head ->
 * greedy argmax per token (p2 "Architecture et structure du code": sampler).
 * READING: the embedding row is the decoded row `token` of tok_emb.
 * logits ([M][vocab]), margin ([M]) and hidden ([M][hidden], the final
 * residual stream before the output norm) may be NULL.
 *
 * Layer skip (p1 feature list and roadmap phase 3: layers picked by cosine
 * similarity are left out of the pass):
 *  - skip (NULL or [n_layer]): a layer with skip[l] != 0 is not run; the
 *    residual stream goes on to the next layer unchanged.
 *  - cosine (NULL or [M][n_layer]): cosine[i][l] receives the cosine
 *    similarity of token i's residual stream entering layer l and leaving
 *    it, x_in . x_out / (|x_in| |x_out|), for every layer that runs; entries
 *    of skipped layers are not written.
 * READING: the similarity is taken on the residual stream itself (no norm
 * applied), per token. */
void or_decode_ex(const or_model* m, const int32_t* tokens, int M, int64_t pos, const uint8_t* skip,
                  int32_t* next, double* logits, double* margin, double* hidden, double* cosine) {
  const int H = m->cfg.hidden;
  int qk = or_block_elems(m->tok_emb.fmt), bb = or_block_bytes(m->tok_emb.fmt);
  int64_t rb = (int64_t)H / qk * bb;
  double* x = (double*)malloc(sizeof(double) * (size_t)M * H);
  double* x_in = (double*)malloc(sizeof(double) * (size_t)M * H);
  double* xn = (double*)malloc(sizeof(double) * H);
  double* lg = (double*)malloc(sizeof(double) * (size_t)m->vocab);
  for (int i = 0; i < M; ++i) or_dequant_row(m->tok_emb.fmt, m->tok_emb.data + (int64_t)tokens[i] * rb, H, x + (int64_t)i * H);
  for (int l = 0; l < m->n_layer; ++l) {
    if (skip && skip[l]) continue;
    memcpy(x_in, x, sizeof(double) * (size_t)M * H);
    or_layer(&m->cfg, &m->layers[l], x, M, pos);
    if (!cosine) continue;
    for (int i = 0; i < M; ++i) {
      const double* a = x_in + (int64_t)i * H;
      const double* b = x + (int64_t)i * H;
      double ab = 0.0, aa = 0.0, bb2 = 0.0;
      for (int r = 0; r < H; ++r) {
        ab += a[r] * b[r];
        aa += a[r] * a[r];
        bb2 += b[r] * b[r];
      }
      cosine[(int64_t)i * m->n_layer + l] = ab / (sqrt(aa) * sqrt(bb2));
    }
  }
  if (hidden) memcpy(hidden, x, sizeof(double) * (size_t)M * H);
  for (int i = 0; i < M; ++i) {
    or_rmsnorm(x + (int64_t)i * H, m->out_norm, H, m->cfg.rms_eps, xn);
    or_gemv(m->lm_head.fmt, m->lm_head.data, xn, lg, m->vocab, H);
    double mg;
    next[i] = (int32_t)or_argmax(lg, m->vocab, &mg);
    if (margin) margin[i] = mg;
    if (logits) memcpy(logits + (int64_t)i * m->vocab, lg, sizeof(double) * (size_t)m->vocab);
  }
  free(x); free(x_in); free(xn); free(lg);
}

/* or_decode_ex with every layer run and no similarities. */
void or_decode(const or_model* m, const int32_t* tokens, int M, int64_t pos, int32_t* next,
               double* logits, double* margin, double* hidden) {
  or_decode_ex(m, tokens, M, pos, NULL, next, logits, margin, hidden, NULL);
}

/* Which layers to skip: the n_skip layers l in [first, last) whose score[l]
 * (a layer's mean input/output cosine similarity over calibration tokens) is
 * largest, since those change the residual stream least (p1 feature list:
 * 20 of 80 layers skipped by cosine similarity).  Picked one at a time, each
 * the largest remaining score, the lower index among equal scores.  mask[l]
 * is 1 for a picked layer and 0 for every other.  Returns 0, or -1 when the
 * range or count is impossible or an eligible score is NaN.
 * READING: the pages give the criterion and the count only; the eligible
 * range (so that e.g. the first and last layers can be kept) and the tie
 * rule are this oracle's. */
int or_select_skip(const double* score, int n_layer, int n_skip, int first, int last, uint8_t* mask) {
  if (n_layer < 0 || first < 0 || first > last || last > n_layer || n_skip < 0 || n_skip > last - first) return -1;
  for (int l = first; l < last; ++l)
    if (isnan(score[l])) return -1;
  for (int l = 0; l < n_layer; ++l) mask[l] = 0;
  for (int k = 0; k < n_skip; ++k) {
    int best = -1;
    for (int l = first; l < last; ++l)
      if (!mask[l] && (best < 0 || score[l] > score[best])) best = l;
    mask[best] = 1;
  }
  return 0;
}
