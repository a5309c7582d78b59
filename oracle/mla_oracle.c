/*
 * mla_oracle.c -- plain, single-threaded CPU reference of the dual-path
 * low-bit MLA cache (writer + decode attention).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark load it.  It shares no code, header, table or constant with
 * the GPU path.
 *
 * What it follows (pages: QuantMLA listing = "QuantMLA" page, RAQ-MLA listing
 * = "RAQ-MLA" page):
 *   - RAQ-MLA, appendix Table 5 (quantizer configuration): latent c_KV in
 *     2-bit (4 levels) or 4-bit (16 levels) codes, per token, groups of 128
 *     channels, FP16 scale and minimum per group, per-token clipping at the
 *     0.94 quantile of |x| for the 2-bit latent; positional key k_R in 4-bit
 *     codes per channel within a cache page, FP16 scale and minimum per
 *     (channel, page), no clipping; effective bits 2 + 32/128 and 4 + 32/P.
 *   - QuantMLA, Figure 8 caption (native mixed-precision execution): a packed
 *     copy of every incoming token; BF16 copies of protected sink and recent
 *     tokens; protected tokens attend from BF16, the rest from dequantized
 *     codes; a token leaving the recent window switches to its existing packed
 *     copy; one softmax over all valid tokens; the reconstructed content tile
 *     is used both for matching and for latent aggregation.
 *   - QuantMLA, Figure 5 caption and Table 10 caption: the sink4/local128
 *     protection policy.
 *   - RAQ-MLA abstract and Figure 4 caption: the latent supplies the values
 *     and, with absorbed queries, score = q_lat . c_KV + q_rope . k_R.
 *
 * Where the pages leave a step open the reading taken is written next to the
 * code (asymmetric min/scale form, directed FP16 rounding of the metadata,
 * round-half-even codes, linear-interpolation quantile, token-major packing).
 *
 * Precision: the quantizer runs in IEEE fp32 with every operation separately
 * rounded (build with -ffp-contract=off, no fast-math), because the code
 * decision must be taken in the same precision as the GPU writer.  The decode
 * runs in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int32_t latent_dim;   /* c_KV channels (512) */
  int32_t rope_dim;     /* k_R channels (64) */
  int32_t page_size;    /* P tokens per cache page */
  int32_t latent_bits;  /* 2 or 4 */
  int32_t rope_bits;    /* 4 */
  int32_t latent_group; /* 128 channels per latent group */
  double latent_clip_q; /* quantile for |x| clipping; 0 = no clipping */
  int32_t sink;         /* protected leading tokens */
  int32_t local;        /* protected recent-window tokens */
} orc_layout;

/* ------------------------------------------------------------------ */
/* Byte layout of one cache page (our reading; the pages give only the
 * per-element totals of RAQ-MLA Table 5):
 *   [latent codes  : P rows x (latent_dim*latent_bits/8) bytes, token-major]
 *   [latent meta   : P rows x groups x (fp16 scale, fp16 min)]
 *   [rope codes    : P rows x (rope_dim*rope_bits/8) bytes, token-major]
 *   [rope meta     : rope_dim fp16 scales, then rope_dim fp16 minimums]
 * Inside a code row, channel c sits in byte (c*bits)/8 at bit offset
 * (c*bits)%8, lower channels in lower bits. */
typedef struct {
  int64_t lat_row, lat_codes_off, lat_meta_off, rope_row, rope_codes_off,
      rope_meta_off, page_bytes;
  int32_t groups;
} orc_geom;

static orc_geom geom_of(const orc_layout* L) {
  orc_geom g;
  int64_t P = L->page_size;
  g.groups = L->latent_dim / L->latent_group;
  g.lat_row = (int64_t)L->latent_dim * L->latent_bits / 8;
  g.rope_row = (int64_t)L->rope_dim * L->rope_bits / 8;
  g.lat_codes_off = 0;
  g.lat_meta_off = P * g.lat_row;
  g.rope_codes_off = g.lat_meta_off + P * g.groups * 4;
  g.rope_meta_off = g.rope_codes_off + P * g.rope_row;
  g.page_bytes = g.rope_meta_off + (int64_t)L->rope_dim * 4;
  return g;
}

int64_t oracle_page_bytes(const orc_layout* L) { return geom_of(L).page_bytes; }

void oracle_page_offsets(const orc_layout* L, int64_t* out6) {
  orc_geom g = geom_of(L);
  out6[0] = g.lat_codes_off;
  out6[1] = g.lat_meta_off;
  out6[2] = g.rope_codes_off;
  out6[3] = g.rope_meta_off;
  out6[4] = g.page_bytes;
  out6[5] = g.lat_row;
}

/* ------------------------------------------------------------------ */
/* bf16 and fp16 by their definitions. */

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16; /* bf16 is the top half of an fp32 */
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* IEEE binary16 value of a bit pattern (finite patterns only are used). */
static double f16_value(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  else
    v = ldexp(1.0 + m / 1024.0, e - 15);
  return sign ? -v : v;
}

/* All finite fp16 values in ascending order (each zero appears once, +0). */
static double g_f16_sorted[63488];
static uint16_t g_f16_bits[63488];
static int g_f16_n = 0;

static int cmp_idx(const void* a, const void* b) {
  double x = f16_value(*(const uint16_t*)a), y = f16_value(*(const uint16_t*)b);
  return (x > y) - (x < y);
}

static void f16_table_init(void) {
  if (g_f16_n) return;
  static uint16_t tmp[63488];
  int n = 0;
  for (uint32_t h = 0; h < 65536; ++h) {
    if (((h >> 10) & 31) == 31) continue; /* inf / nan */
    if (h == 0x8000) continue;            /* -0: kept out, zero is +0 */
    tmp[n++] = (uint16_t)h;
  }
  qsort(tmp, n, sizeof(uint16_t), cmp_idx);
  for (int i = 0; i < n; ++i) {
    g_f16_bits[i] = tmp[i];
    g_f16_sorted[i] = f16_value(tmp[i]);
  }
  g_f16_n = n;
}

/* Largest finite fp16 value <= x (x finite, |x| <= 65504).  Zero results are
 * returned as +0 (inputs never carry -0: see canon_zero). */
uint16_t oracle_f16_round_down(float xf) {
  f16_table_init();
  double x = xf;
  int lo = 0, hi = g_f16_n - 1, ans = 0;
  if (x < g_f16_sorted[0]) return g_f16_bits[0];
  while (lo <= hi) { /* last index with value <= x */
    int mid = (lo + hi) / 2;
    if (g_f16_sorted[mid] <= x) {
      ans = mid;
      lo = mid + 1;
    } else
      hi = mid - 1;
  }
  return g_f16_bits[ans];
}

/* Smallest finite fp16 value >= x. */
uint16_t oracle_f16_round_up(float xf) {
  f16_table_init();
  double x = xf;
  int lo = 0, hi = g_f16_n - 1, ans = g_f16_n - 1;
  if (x > g_f16_sorted[g_f16_n - 1]) return g_f16_bits[g_f16_n - 1];
  while (lo <= hi) { /* first index with value >= x */
    int mid = (lo + hi) / 2;
    if (g_f16_sorted[mid] >= x) {
      ans = mid;
      hi = mid - 1;
    } else
      lo = mid + 1;
  }
  return g_f16_bits[ans];
}

double oracle_f16_value(uint16_t h) { return f16_value(h); }

/* -0 is read as +0 so that a group minimum is never a signed zero whose sign
 * would depend on the order of a reduction. */
static float canon_zero(float x) { return x == 0.0f ? 0.0f : x; }

/* ------------------------------------------------------------------ */
/* Clipping of one 2-bit latent token at the 0.94 quantile of its absolute
 * values (RAQ-MLA Table 5, clipping row).  Reading: the quantile is taken over all channels
 * of the token, with linear interpolation between order statistics at
 * position h = (n-1) q: c = a[lo] + frac * (a[lo+1] - a[lo]), lo = floor(h),
 * evaluated as three separately rounded fp32 operations. */

static int cmp_float(const void* a, const void* b) {
  float x = *(const float*)a, y = *(const float*)b;
  return (x > y) - (x < y);
}

void oracle_quantile_params(int32_t n, double q, int32_t* lo, int32_t* hi,
                            float* frac) {
  double h = (double)(n - 1) * q;
  int32_t l = (int32_t)floor(h);
  if (l > n - 1) l = n - 1;
  if (l < 0) l = 0;
  *lo = l;
  *hi = l + 1 < n ? l + 1 : n - 1;
  *frac = (float)(h - (double)l);
}

float oracle_clip_value(const float* x, int32_t n, double q) {
  float* a = (float*)malloc(sizeof(float) * n);
  for (int i = 0; i < n; ++i) a[i] = fabsf(x[i]);
  qsort(a, n, sizeof(float), cmp_float);
  int32_t lo, hi;
  float frac;
  oracle_quantile_params(n, q, &lo, &hi, &frac);
  float d = a[hi] - a[lo];
  float p = frac * d;
  float c = a[lo] + p;
  free(a);
  return c;
}

/* ------------------------------------------------------------------ */
/* Asymmetric min/scale quantizer of one group (RAQ-MLA Table 5: FP16 scale
 * and minimum per group).  Readings:
 *   min_h = the fp16 value nearest below the group minimum,
 *   s     = (max - min_h) / levels in fp32,  s_h = the fp16 value nearest
 *           above s  (so the grid min_h + k s_h, k = 0..levels, covers the
 *           group),
 *   code  = round-half-even((x - min_h) / s_h) clamped to [0, levels]; a
 *           zero scale gives code 0.
 * Dequantization is x_hat = code * s_h + min_h. */
void oracle_quantize_group(const float* x, int32_t n, int32_t stride,
                           int32_t levels, uint16_t* scale_h, uint16_t* min_h,
                           uint8_t* codes) {
  float mn = x[0], mx = x[0];
  for (int i = 1; i < n; ++i) {
    float v = x[(int64_t)i * stride];
    if (v < mn) mn = v;
    if (v > mx) mx = v;
  }
  uint16_t mh = oracle_f16_round_down(mn);
  float minf = (float)f16_value(mh);
  float span = mx - minf;
  float s = span / (float)levels;
  uint16_t sh = oracle_f16_round_up(s);
  float sf = (float)f16_value(sh);
  for (int i = 0; i < n; ++i) {
    float v = x[(int64_t)i * stride];
    int code = 0;
    if (sf > 0.0f) {
      float t = (v - minf) / sf;
      float r = rintf(t);
      if (r < 0.0f) r = 0.0f;
      if (r > (float)levels) r = (float)levels;
      code = (int)r;
    }
    codes[i] = (uint8_t)code;
  }
  *scale_h = sh;
  *min_h = mh;
}

/* Place code `code` of channel `c` into a packed row. */
static void put_code(uint8_t* row, int c, int bits, int code) {
  int bit = c * bits;
  row[bit / 8] |= (uint8_t)(code << (bit % 8));
}

static int get_code(const uint8_t* row, int c, int bits) {
  int bit = c * bits;
  return (row[bit / 8] >> (bit % 8)) & ((1 << bits) - 1);
}

void oracle_pack_row(const uint8_t* codes, int32_t n, int32_t bits,
                     uint8_t* row) {
  memset(row, 0, (size_t)n * bits / 8);
  for (int c = 0; c < n; ++c) put_code(row, c, bits, codes[c]);
}

void oracle_unpack_row(const uint8_t* row, int32_t n, int32_t bits,
                       uint8_t* codes) {
  for (int c = 0; c < n; ++c) codes[c] = (uint8_t)get_code(row, c, bits);
}

static void put_f16(uint8_t* p, uint16_t h) { memcpy(p, &h, 2); }
static uint16_t get_f16(const uint8_t* p) {
  uint16_t h;
  memcpy(&h, p, 2);
  return h;
}

/* Quantize one latent token into its page row: optional clipping, then one
 * quantizer per group. */
static void write_latent_token(const orc_layout* L, const orc_geom* G,
                               const uint16_t* src, uint8_t* page, int slot) {
  int D = L->latent_dim, levels = (1 << L->latent_bits) - 1;
  float* x = (float*)malloc(sizeof(float) * D);
  uint8_t* codes = (uint8_t*)malloc(D);
  for (int c = 0; c < D; ++c) x[c] = canon_zero(bf16_to_f32(src[c]));
  if (L->latent_clip_q > 0.0) {
    float cl = oracle_clip_value(x, D, L->latent_clip_q);
    for (int c = 0; c < D; ++c) {
      float v = x[c];
      if (v < -cl) v = -cl;
      if (v > cl) v = cl;
      x[c] = canon_zero(v);
    }
  }
  uint8_t* meta = page + G->lat_meta_off + (int64_t)slot * G->groups * 4;
  for (int g = 0; g < G->groups; ++g) {
    uint16_t sh, mh;
    oracle_quantize_group(x + g * L->latent_group, L->latent_group, 1, levels,
                          &sh, &mh, codes + g * L->latent_group);
    put_f16(meta + g * 4, sh);
    put_f16(meta + g * 4 + 2, mh);
  }
  oracle_pack_row(codes, D, L->latent_bits,
                  page + G->lat_codes_off + (int64_t)slot * G->lat_row);
  free(x);
  free(codes);
}

/* Quantize the positional key of a completed page, per channel over its P
 * tokens (RAQ-MLA Table 5: per channel within a cache page, no clipping). */
static void finalize_rope_page(const orc_layout* L, const orc_geom* G,
                               const uint16_t* tail, uint8_t* page) {
  int P = L->page_size, R = L->rope_dim, levels = (1 << L->rope_bits) - 1;
  float* x = (float*)malloc(sizeof(float) * P * R);
  uint8_t* codes = (uint8_t*)malloc((size_t)P * R);
  uint8_t* col = (uint8_t*)malloc(P);
  for (int t = 0; t < P; ++t)
    for (int c = 0; c < R; ++c)
      x[t * R + c] = canon_zero(bf16_to_f32(tail[(int64_t)t * R + c]));
  uint8_t* meta = page + G->rope_meta_off;
  for (int c = 0; c < R; ++c) {
    uint16_t sh, mh;
    oracle_quantize_group(x + c, P, R, levels, &sh, &mh, col);
    for (int t = 0; t < P; ++t) codes[t * R + c] = col[t];
    put_f16(meta + 2 * c, sh);
    put_f16(meta + 2 * R + 2 * c, mh);
  }
  for (int t = 0; t < P; ++t)
    oracle_pack_row(codes + t * R, R, L->rope_bits,
                    page + G->rope_codes_off + (int64_t)t * G->rope_row);
  free(x);
  free(codes);
  free(col);
}

/* ------------------------------------------------------------------ */
/* Writer: appends new tokens of each sequence in order (QuantMLA Figure 8:
 * a packed copy of every incoming token, BF16 retention of protected
 * tokens).  State per sequence:
 *   sink[b][t]            BF16 row [c_KV | k_R] of token t < sink,
 *   ring[b][t % local]    BF16 row of the most recent tokens,
 *   tail[b][t % P]        BF16 k_R of the tokens of the page being filled;
 *                         when the page's last slot is written its k_R is
 *                         quantized per channel (finalize_rope_page).
 * Rows of c_kv / k_r are bf16; new tokens of sequence b are rows
 * cu_new[b] .. cu_new[b+1]-1, at positions seqlens_before[b] + i. */
int oracle_write(const orc_layout* L, const uint16_t* c_kv,
                 const uint16_t* k_r, const int32_t* cu_new,
                 const int32_t* seqlens_before, int32_t batch,
                 const int32_t* block_table, int32_t max_pages, uint8_t* pool,
                 uint16_t* sink_buf, uint16_t* ring_buf, uint16_t* tail_buf) {
  orc_geom G = geom_of(L);
  int P = L->page_size, D = L->latent_dim, R = L->rope_dim, W = D + R;
  for (int b = 0; b < batch; ++b) {
    int n_new = cu_new[b + 1] - cu_new[b];
    for (int i = 0; i < n_new; ++i) {
      int64_t row = cu_new[b] + i;
      int t = seqlens_before[b] + i;
      int pidx = t / P, slot = t % P;
      if (pidx >= max_pages) return -1;
      uint8_t* page = pool + (int64_t)block_table[(int64_t)b * max_pages + pidx] *
                                 G.page_bytes;
      const uint16_t* xl = c_kv + row * D;
      const uint16_t* xr = k_r + row * R;
      write_latent_token(L, &G, xl, page, slot);
      if (t < L->sink) {
        uint16_t* dst = sink_buf + ((int64_t)b * L->sink + t) * W;
        memcpy(dst, xl, 2 * D);
        memcpy(dst + D, xr, 2 * R);
      }
      if (L->local > 0) {
        uint16_t* dst = ring_buf + ((int64_t)b * L->local + t % L->local) * W;
        memcpy(dst, xl, 2 * D);
        memcpy(dst + D, xr, 2 * R);
      }
      uint16_t* tail = tail_buf + (int64_t)b * P * R;
      memcpy(tail + (int64_t)slot * R, xr, 2 * R);
      if (slot == P - 1) finalize_rope_page(L, &G, tail, page);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Reconstruct token j of sequence b (fp64, latent_dim + rope_dim values)
 * as the attention reads it (QuantMLA Figure 8):
 *   j < sink or j >= Lb - local  -> the BF16 copy (sink row / ring slot),
 *   otherwise                    -> dequantized latent codes; the k_R of a
 *                                   completed page from its codes, of the
 *                                   page still being filled from the BF16
 *                                   tail (it has no codes yet).
 * Returns 0 for a packed latent, 1 for a BF16 row. */
int oracle_read_token(const orc_layout* L, const uint8_t* pool,
                      const int32_t* bt_row, const uint16_t* sink_buf,
                      const uint16_t* ring_buf, const uint16_t* tail_buf,
                      int32_t b, int32_t Lb, int32_t j, double* out) {
  orc_geom G = geom_of(L);
  int P = L->page_size, D = L->latent_dim, R = L->rope_dim, W = D + R;
  const uint16_t* bf = NULL;
  if (j < L->sink)
    bf = sink_buf + ((int64_t)b * L->sink + j) * W;
  else if (L->local > 0 && j >= Lb - L->local)
    bf = ring_buf + ((int64_t)b * L->local + j % L->local) * W;
  if (bf) {
    for (int c = 0; c < W; ++c) out[c] = bf16_to_f32(bf[c]);
    return 1;
  }
  int pidx = j / P, slot = j % P;
  const uint8_t* page = pool + (int64_t)bt_row[pidx] * G.page_bytes;
  const uint8_t* crow = page + G.lat_codes_off + (int64_t)slot * G.lat_row;
  const uint8_t* meta = page + G.lat_meta_off + (int64_t)slot * G.groups * 4;
  for (int c = 0; c < D; ++c) {
    int g = c / L->latent_group;
    double s = f16_value(get_f16(meta + 4 * g)), m = f16_value(get_f16(meta + 4 * g + 2));
    out[c] = get_code(crow, c, L->latent_bits) * s + m;
  }
  int page_complete = (int64_t)(pidx + 1) * P <= Lb;
  if (page_complete) {
    const uint8_t* rrow = page + G.rope_codes_off + (int64_t)slot * G.rope_row;
    const uint8_t* rm = page + G.rope_meta_off;
    for (int c = 0; c < R; ++c) {
      double s = f16_value(get_f16(rm + 2 * c)), m = f16_value(get_f16(rm + 2 * R + 2 * c));
      out[D + c] = get_code(rrow, c, L->rope_bits) * s + m;
    }
  } else {
    const uint16_t* tail = tail_buf + (int64_t)b * P * R + (int64_t)slot * R;
    for (int c = 0; c < R; ++c) out[D + c] = bf16_to_f32(tail[c]);
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Decode attention with absorbed queries (RAQ-MLA abstract / Figure 4;
 * QuantMLA Figure 8), fp64, per (sequence, head):
 *   z_j  = scale * (q_lat . c_hat_j + q_rope . k_hat_j),  j = 0..Lb-1
 *   out  = sum_j exp(z_j - max z) c_hat_j / sum_j exp(z_j - max z)
 *   lse  = max z + log(sum_j exp(z_j - max z))
 * Lb = 0 gives out = 0 and lse = -inf.  q rows are bf16 [B][H][dim]. */
void oracle_decode(const orc_layout* L, const uint16_t* q_lat,
                   const uint16_t* q_rope, int32_t batch, int32_t heads,
                   double scale, const uint8_t* pool, const int32_t* block_table,
                   int32_t max_pages, const int32_t* seqlens,
                   const uint16_t* sink_buf, const uint16_t* ring_buf,
                   const uint16_t* tail_buf, double* out, double* lse) {
  int D = L->latent_dim, R = L->rope_dim, W = D + R;
  double* tok = (double*)malloc(sizeof(double) * W);
  double* q = (double*)malloc(sizeof(double) * (size_t)heads * W);
  for (int b = 0; b < batch; ++b) {
    int Lb = seqlens[b];
    const int32_t* bt = block_table + (int64_t)b * max_pages;
    double* z = (double*)malloc(sizeof(double) * (size_t)heads * (Lb > 0 ? Lb : 1));
    for (int h = 0; h < heads; ++h) {
      for (int c = 0; c < D; ++c) q[h * W + c] = bf16_to_f32(q_lat[((int64_t)b * heads + h) * D + c]);
      for (int c = 0; c < R; ++c) q[h * W + D + c] = bf16_to_f32(q_rope[((int64_t)b * heads + h) * R + c]);
    }
    /* pass 1: logits */
    for (int j = 0; j < Lb; ++j) {
      oracle_read_token(L, pool, bt, sink_buf, ring_buf, tail_buf, b, Lb, j, tok);
      for (int h = 0; h < heads; ++h) {
        double acc = 0.0;
        for (int c = 0; c < W; ++c) acc += q[h * W + c] * tok[c];
        z[(int64_t)h * Lb + j] = scale * acc;
      }
    }
    double* o = out + (int64_t)b * heads * D;
    memset(o, 0, sizeof(double) * (size_t)heads * D);
    if (Lb == 0) {
      for (int h = 0; h < heads; ++h) lse[(int64_t)b * heads + h] = -INFINITY;
      free(z);
      continue;
    }
    double* mx = (double*)malloc(sizeof(double) * heads);
    double* sum = (double*)malloc(sizeof(double) * heads);
    for (int h = 0; h < heads; ++h) {
      double m = -INFINITY, s = 0.0;
      for (int j = 0; j < Lb; ++j) m = fmax(m, z[(int64_t)h * Lb + j]);
      for (int j = 0; j < Lb; ++j) s += exp(z[(int64_t)h * Lb + j] - m);
      mx[h] = m;
      sum[h] = s;
    }
    /* pass 2: latent aggregation with the same reconstructed tokens */
    for (int j = 0; j < Lb; ++j) {
      oracle_read_token(L, pool, bt, sink_buf, ring_buf, tail_buf, b, Lb, j, tok);
      for (int h = 0; h < heads; ++h) {
        double p = exp(z[(int64_t)h * Lb + j] - mx[h]) / sum[h];
        double* oh = o + (int64_t)h * D;
        for (int c = 0; c < D; ++c) oh[c] += p * tok[c];
      }
    }
    for (int h = 0; h < heads; ++h) lse[(int64_t)b * heads + h] = mx[h] + log(sum[h]);
    free(mx);
    free(sum);
    free(z);
  }
  free(tok);
  free(q);
}

/* ------------------------------------------------------------------ */
/* Decode over a plain BF16 paged cache: the baseline the low-bit cache is
 * measured against (QuantMLA, Table 9 caption: BF16 attention with native
 * partitioning).  Reading taken: the cache keeps every token's pre-
 * quantization row (c_KV 512 then k_R 64, bf16) at page
 * block_table[b][j / P], slot j % P of a pool [pages][P][576]; the attention
 * is the same as oracle_decode's with every token read from that row:
 *   z_j = scale * (q_lat . c_j + q_rope . k_j)
 *   out = sum_j exp(z_j - max z) c_j / sum_j exp(z_j - max z)
 *   lse = max z + log(sum_j exp(z_j - max z)),  fp64.
 * Lb = 0 gives out = 0 and lse = -inf. */
void oracle_decode_bf16(const uint16_t* q_lat, const uint16_t* q_rope, int32_t batch, int32_t heads,
                        double scale, const uint16_t* pool, int32_t page_size,
                        const int32_t* block_table, int32_t max_pages, const int32_t* seqlens,
                        double* out, double* lse) {
  const int D = 512, R = 64, W = D + R;
  double* q = (double*)malloc(sizeof(double) * (size_t)W);
  for (int b = 0; b < batch; ++b) {
    int Lb = seqlens[b];
    const int32_t* bt = block_table + (int64_t)b * max_pages;
    double* z = (double*)malloc(sizeof(double) * (size_t)(Lb > 0 ? Lb : 1));
    for (int h = 0; h < heads; ++h) {
      for (int c = 0; c < D; ++c) q[c] = bf16_to_f32(q_lat[((int64_t)b * heads + h) * D + c]);
      for (int c = 0; c < R; ++c) q[D + c] = bf16_to_f32(q_rope[((int64_t)b * heads + h) * R + c]);
      double* o = out + ((int64_t)b * heads + h) * D;
      memset(o, 0, sizeof(double) * D);
      if (Lb == 0) {
        lse[(int64_t)b * heads + h] = -INFINITY;
        continue;
      }
      double m = -INFINITY;
      for (int j = 0; j < Lb; ++j) {
        const uint16_t* row = pool + ((int64_t)bt[j / page_size] * page_size + j % page_size) * W;
        double acc = 0.0;
        for (int c = 0; c < W; ++c) acc += q[c] * bf16_to_f32(row[c]);
        z[j] = scale * acc;
        m = fmax(m, z[j]);
      }
      double sum = 0.0;
      for (int j = 0; j < Lb; ++j) sum += exp(z[j] - m);
      for (int j = 0; j < Lb; ++j) {
        const uint16_t* row = pool + ((int64_t)bt[j / page_size] * page_size + j % page_size) * W;
        double p = exp(z[j] - m) / sum;
        for (int c = 0; c < D; ++c) o[c] += p * bf16_to_f32(row[c]);
      }
      lse[(int64_t)b * heads + h] = m + log(sum);
    }
    free(z);
  }
  free(q);
}

/* ------------------------------------------------------------------ */
/* Array helpers for the tests' pins. */
void oracle_f16_round_down_n(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_round_down(x[i]);
}
void oracle_f16_round_up_n(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_round_up(x[i]);
}

/* ------------------------------------------------------------------ */
/* Latent transform before the cache write (RAQ-MLA, Figure 4 caption: A_c
 * acts on the latent before it is quantized; appendix Table 9: applied inside
 * the write kernel).  Reading taken: y = A_c x with A_c stored row-major
 * [out][in] in bf16; each output is an fp32 fused multiply-add chain over the
 * inputs in ascending order, rounded once to bf16 (nearest, ties to even),
 * and the writer then caches y exactly as it caches an untransformed row.
 * The pages do not fix the transform's precision, so the decision is taken
 * in the GPU writer's: single-precision fma in input order. */

static uint16_t f32_to_bf16_rne(float f) {
  /* keep the top 16 bits of the fp32 pattern, rounding the 16 dropped bits
   * to nearest with ties to the even kept pattern (finite inputs) */
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint32_t dropped = u & 0xFFFFu, kept = u >> 16;
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) return (uint16_t)(kept + 1u);
  return (uint16_t)kept;
}

/* y[t][c] = bf16(fma chain over k of A[c][k] * x[t][k]) for t < n_tokens. */
void oracle_transform(const uint16_t* a_c, const uint16_t* x, int64_t n_tokens, int32_t dim, uint16_t* y) {
  for (int64_t t = 0; t < n_tokens; ++t) {
    for (int32_t c = 0; c < dim; ++c) {
      float acc = 0.0f;
      for (int32_t k = 0; k < dim; ++k)
        acc = fmaf(bf16_to_f32(a_c[(int64_t)c * dim + k]), bf16_to_f32(x[t * dim + k]), acc);
      y[t * dim + c] = f32_to_bf16_rne(acc);
    }
  }
}
