// Small kernels of the forward pass: RoPE tables, embedding gather, row
// RMSNorm, the prefill QK-norm / RoPE / KV-cache write, the fp32-weight GEMV,
// row argmax and weight-format conversions.
#include "common.h"
#include "kernels.h"

namespace dpk {

namespace {

// cos/sin of pos * theta^(-2i/d), evaluated in double on the device, stored fp32.
__global__ void rope_table_kernel(float* cos_t, float* sin_t, int max_seq, int d, double theta) {
  const int hd2 = d / 2;
  const size_t n = (size_t)max_seq * hd2;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < n; idx += (size_t)gridDim.x * blockDim.x) {
    const int pos = (int)(idx / hd2), i = (int)(idx % hd2);
    const double inv = pow(theta, -2.0 * (double)i / (double)d);
    const double ang = (double)pos * inv;
    cos_t[idx] = (float)cos(ang);
    sin_t[idx] = (float)sin(ang);
  }
}

// one workgroup per row; token from RowParam (or ids_dev when given)
__global__ void embed_kernel(int H, int fmt, const void* table, const void* scp, const uint16_t* bi,
                             const RowParam* rp, const int32_t* ids_dev, int vocab, float* h, float* rs,
                             float eps, int* err_flag, float* sq) {
  __shared__ float red[32];
  const int m = blockIdx.x;
  int tok = ids_dev ? ids_dev[m] : rp[m].token;
  if (tok < 0 || tok >= vocab) {
    if (threadIdx.x == 0 && err_flag) atomicOr(err_flag, 1);
    tok = 0;
  }
  const uint16_t* sc = (const uint16_t*)scp;
  float ss = 0.f;
  for (int k = threadIdx.x; k < H; k += blockDim.x) {
    float v;
    if (fmt == W_F32) {
      v = ((const float*)table)[(size_t)tok * H + k];
    } else if (fmt == W_BF16) {
      v = bf16_to_f32(((const uint16_t*)table)[(size_t)tok * H + k]);
    } else if (fmt == W_I8) {  // int8 per output row: w = s * q
      v = bf16_to_f32(sc[tok]) * (float)((const int8_t*)table)[(size_t)tok * H + k];
    } else if (fmt == W_Q8) {  // int8 in blocks of 32 with an fp32 scale each
      v = ((const float*)scp)[(size_t)tok * (H / 32) + k / 32] * (float)((const int8_t*)table)[(size_t)tok * H + k];
    } else if (fmt == W_Q40) {  // 4-bit blocks of 32 around 8, fp16 scale; byte j: codes j, j + 16
      const int i = k & 31;
      const uint8_t b = ((const uint8_t*)table)[(size_t)tok * (H / 2) + (k / 32) * 16 + (i & 15)];
      const int c = i < 16 ? (b & 0xF) : (b >> 4);
      v = (float)__builtin_bit_cast(_Float16, sc[(size_t)tok * (H / 32) + k / 32]) * (float)(c - 8);
    } else {  // MLX 4-bit: w = s * c + b, group 64 along the row
      const uint32_t word = ((const uint32_t*)table)[(size_t)tok * (H / 8) + k / 8];
      const float c = (float)((word >> (4 * (k & 7))) & 0xF);
      const size_t g = (size_t)tok * (H / 64) + k / 64;
      v = bf16_to_f32(sc[g]) * c + bf16_to_f32(bi[g]);
    }
    h[(size_t)m * H + k] = v;
    ss += v * v;
  }
  if (rs || sq) {
    ss = block_sum(ss, red);
    if (threadIdx.x == 0 && rs) rs[m] = rsqrtf(ss / (float)H + eps);
    if (threadIdx.x == 0 && sq) sq[m] = ss;
  }
}

// grid (M, ceil(K / 2048)), 256 threads x 8 elements
__global__ void xprep_kernel(int K, const float* x, int ldx, const float* sq_in, int nb, const uint16_t* g, float eps,
                             uint16_t* hi, uint16_t* lo) {
  __shared__ float red[8];
  const int m = blockIdx.x;
  float rs = 1.0f;
  if (sq_in) {
    float s = 0.f;
    for (int b = threadIdx.x; b < nb; b += blockDim.x) s += sq_in[(size_t)m * nb + b];
    s = block_sum(s, red);
    rs = rsqrtf(s / (float)K + eps);
  }
  const int k = (blockIdx.y * blockDim.x + threadIdx.x) * 8;
  if (k >= K) return;
  const float* xp = x + (size_t)m * ldx + k;
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    float v0 = xp[e] * rs, v1 = xp[e + 1] * rs;
    if (g) {
      v0 *= bf16_to_f32(g[k + e]);
      v1 *= bf16_to_f32(g[k + e + 1]);
    }
    uint32_t h0, l0, h1, l1;
    split_bf16(v0, h0, l0);
    split_bf16(v1, h1, l1);
    h[e / 2] = h0 | (h1 << 16);
    l[e / 2] = l0 | (l1 << 16);
  }
  // 8 consecutive columns stay inside one 32-column block of the layout
  *(uint4*)(hi + xg_index(m, k)) = make_uint4(h[0], h[1], h[2], h[3]);
  *(uint4*)(lo + xg_index(m, k)) = make_uint4(l[0], l[1], l[2], l[3]);
}

__global__ void rmsnorm_rows_kernel(int H, const float* x, int ldx, const void* g, int g_is_f32, float eps,
                                    void* y, int y_is_f16, int ldy) {
  __shared__ float red[32];
  const int m = blockIdx.x;
  const float* xr = x + (size_t)m * ldx;
  float ss = 0.f;
  for (int k = threadIdx.x; k < H; k += blockDim.x) ss += xr[k] * xr[k];
  ss = block_sum(ss, red);
  const float r = rsqrtf(ss / (float)H + eps);
  for (int k = threadIdx.x; k < H; k += blockDim.x) {
    const float gk = g_is_f32 ? ((const float*)g)[k] : bf16_to_f32(((const uint16_t*)g)[k]);
    const float v = xr[k] * r * gk;
    if (y_is_f16 == 2) {  // fp16 hi in [0, H), fp16 lo = v - hi in [H, 2H)
      const _Float16 hi = (_Float16)v;
      ((_Float16*)y)[(size_t)m * ldy + k] = hi;
      ((_Float16*)y)[(size_t)m * ldy + H + k] = (_Float16)(v - (float)hi);
    } else if (y_is_f16) {
      ((_Float16*)y)[(size_t)m * ldy + k] = (_Float16)v;
    } else {
      ((float*)y)[(size_t)m * ldy + k] = v;
    }
  }
}

// Prefill variant of rmsnorm_rows (bf16 gain, fp16 output, H = NV * 2048):
// each thread holds 8 consecutive columns per 2048 in registers (one read of
// the row), 16-byte loads and stores.  mode 1: fp16; 2: fp16 hi in [0, H),
// lo = v - hi in [H, 2H).
template <int NV>
__global__ __launch_bounds__(256) void rmsnorm_vec_kernel(int H, const float* x, int ldx, const uint16_t* g,
                                                         float eps, _Float16* y, int mode, int ldy) {
  __shared__ float red[8];
  const int m = blockIdx.x, tid = threadIdx.x;
  const float* xr = x + (size_t)m * ldx;
  float v[NV][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int k = (j * 256 + tid) * 8;
    const float4 a = *(const float4*)(xr + k), b = *(const float4*)(xr + k + 4);
    v[j][0] = a.x; v[j][1] = a.y; v[j][2] = a.z; v[j][3] = a.w;
    v[j][4] = b.x; v[j][5] = b.y; v[j][6] = b.z; v[j][7] = b.w;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += v[j][e] * v[j][e];
  }
  ss = block_sum(ss, red);
  const float r = rsqrtf(ss / (float)H + eps);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int k = (j * 256 + tid) * 8;
    const uint4 gw = *(const uint4*)(g + k);
    const uint32_t gg[4] = {gw.x, gw.y, gw.z, gw.w};
    f16x8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float gk = (e & 1) ? bf16hi_to_f32(gg[e / 2]) : bf16lo_to_f32(gg[e / 2]);
      const float t = v[j][e] * r * gk;
      hi[e] = (_Float16)t;
      lo[e] = (_Float16)(t - (float)hi[e]);
    }
    _Float16* yr = y + (size_t)m * ldy;
    *(f16x8*)(yr + k) = hi;
    if (mode == 2) *(f16x8*)(yr + H + k) = lo;
  }
}

// Prefill variant of qk_rope_kv (fp16 hi / lo q planes, bf16 gains, d = 128,
// rows at consecutive positions of one sequence): grid (ceil(M / 64), n_heads
// + 2 n_kv), 4 waves of 16 rows each.  A value head goes through LDS so that
// its transposed slab rows are written 64 positions at a time.
__global__ __launch_bounds__(256) void qk_rope_kv_rows_kernel(const float* qkv, int M, int n_heads, int n_kv,
                                                            const uint16_t* qn, const uint16_t* kn, float eps,
                                                            const float* rope_cos, const float* rope_sin,
                                                            const RowParam* rp, _Float16* q_out, KVDesc kv,
                                                            int layer) {
  constexpr int D = 128, HD = 64;
  __shared__ _Float16 vt[D][64 + 2];
  const int blk = blockIdx.x, hh = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ld = (n_heads + 2 * n_kv) * D;
  const int m0 = blk * 64;
  const int rows = min(64, M - m0);
  const RowParam r0 = rp[m0];
  if (hh >= n_heads + n_kv) {  // v head -> V^T slab
    const int vh = hh - n_heads - n_kv;
    if (kv.i8) {  // int8 cache: one wave per position (codes + scale)
      for (int rr = wave; rr < rows; rr += 4) {
        const float* src = qkv + (size_t)(m0 + rr) * ld + (size_t)hh * D;
        kv_put_i8(kv, r0.seq, layer, 1, vh, r0.pos + rr, src[lane], src[lane + HD], lane);
      }
      return;
    }
    for (int i = tid; i < rows * D; i += 256) {
      const int rr = i / D, e = i % D;
      vt[e][rr] = (_Float16)qkv[(size_t)(m0 + rr) * ld + (size_t)hh * D + e];
    }
    __syncthreads();
    _Float16* vb = (_Float16*)kv.base + kv_slab(kv, r0.seq, layer, 1, vh);
    for (int i = tid; i < D * 64; i += 256) {
      const int e = i / 64, rr = i % 64;
      if (rr < rows) vb[(size_t)e * kv.max_seq + r0.pos + rr] = vt[e][rr];
    }
    return;
  }
  const bool is_q = hh < n_heads;
  const uint16_t* g = is_q ? qn : kn;
  // this wave's 16 rows loaded first (clamped: rows past M repeat the last)
  float av[16], bv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float* src = qkv + (size_t)(m0 + min(wave + 4 * i, rows - 1)) * ld + (size_t)hh * D;
    av[i] = src[lane];
    bv[i] = src[lane + HD];
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rr = wave + 4 * i;
    if (rr >= rows) break;
    const int m = m0 + rr;
    const float a = av[i], b = bv[i];
    float scale = 1.f;
    if (g) scale = rsqrtf(wave_sum(a * a + b * b) / (float)D + eps);
    float x1 = a * scale, x2 = b * scale;
    if (g) {
      x1 *= bf16_to_f32(g[lane]);
      x2 *= bf16_to_f32(g[lane + HD]);
    }
    const int pos = r0.pos + rr;
    const float c = rope_cos[(size_t)pos * HD + lane], sn = rope_sin[(size_t)pos * HD + lane];
    const float y1 = x1 * c - x2 * sn, y2 = x2 * c + x1 * sn;
    if (is_q) {
      const size_t o = ((size_t)m * n_heads + hh) * D;
      _Float16* qh = q_out;
      _Float16* ql = q_out + (size_t)M * n_heads * D;
      const _Float16 h1 = (_Float16)y1, h2 = (_Float16)y2;
      qh[o + lane] = h1;
      qh[o + lane + HD] = h2;
      ql[o + lane] = (_Float16)(y1 - (float)h1);
      ql[o + lane + HD] = (_Float16)(y2 - (float)h2);
    } else if (kv.i8) {
      kv_put_i8(kv, r0.seq, layer, 0, hh - n_heads, pos, y1, y2, lane);
    } else {
      _Float16* kb = (_Float16*)kv.base + kv_slab(kv, r0.seq, layer, 0, hh - n_heads) + (size_t)pos * D;
      kb[lane] = (_Float16)y1;
      kb[lane + HD] = (_Float16)y2;
    }
  }
}

// grid (M, n_heads + 2*n_kv); one workgroup of 64 threads per (row, head)
__global__ void qk_rope_kv_kernel(const float* qkv, int n_heads, int n_kv, int d, int qk_norm, const void* qn,
                                  const void* kn, int g_is_f32, float eps, const float* rope_cos,
                                  const float* rope_sin, const RowParam* rp, void* q_out, int q_is_f16,
                                  KVDesc kv, int layer) {
  const int m = blockIdx.x, hh = blockIdx.y, lane = threadIdx.x;
  const int ld = (n_heads + 2 * n_kv) * d;
  const float* src = qkv + (size_t)m * ld + (size_t)hh * d;
  const RowParam r = rp[m];
  const int hd2 = d / 2;
  if (hh >= n_heads + n_kv) {  // v head -> V^T slab
    const int vh = hh - n_heads - n_kv;
    if (kv.i8) {  // (d == 128)
      kv_put_i8(kv, r.seq, layer, 1, vh, r.pos, src[lane], src[lane + 64], lane);
      return;
    }
    for (int e = lane; e < d; e += 64) kv_store(kv, kv_offset(kv, r.seq, layer, 1, vh, e, r.pos), src[e]);
    return;
  }
  const bool is_q = hh < n_heads;
  float scale = 1.f;
  if (qk_norm) {
    float ss = 0.f;
    for (int e = lane; e < d; e += 64) ss += src[e] * src[e];
    ss = wave_sum(ss);
    scale = rsqrtf(ss / (float)d + eps);
  }
  const void* g = is_q ? qn : kn;
  for (int e = lane; e < hd2; e += 64) {
    float x1 = src[e] * scale, x2 = src[e + hd2] * scale;
    if (qk_norm && g) {
      if (g_is_f32) {
        x1 *= ((const float*)g)[e];
        x2 *= ((const float*)g)[e + hd2];
      } else {
        x1 *= bf16_to_f32(((const uint16_t*)g)[e]);
        x2 *= bf16_to_f32(((const uint16_t*)g)[e + hd2]);
      }
    }
    const float c = rope_cos[(size_t)r.pos * hd2 + e], s = rope_sin[(size_t)r.pos * hd2 + e];
    const float y1 = x1 * c - x2 * s, y2 = x2 * c + x1 * s;
    if (is_q) {
      const size_t o = ((size_t)m * n_heads + hh) * d;
      if (q_is_f16 == 2) {
        // fp16 hi plane, then the lo plane (y - hi) M * n_heads * d further
        _Float16* qh = (_Float16*)q_out;
        _Float16* ql = qh + (size_t)gridDim.x * n_heads * d;
        const _Float16 h1 = (_Float16)y1, h2 = (_Float16)y2;
        qh[o + e] = h1;
        qh[o + e + hd2] = h2;
        ql[o + e] = (_Float16)(y1 - (float)h1);
        ql[o + e + hd2] = (_Float16)(y2 - (float)h2);
      } else if (q_is_f16) {
        ((_Float16*)q_out)[o + e] = (_Float16)y1;
        ((_Float16*)q_out)[o + e + hd2] = (_Float16)y2;
      } else {
        ((float*)q_out)[o + e] = y1;
        ((float*)q_out)[o + e + hd2] = y2;
      }
    } else if (kv.i8) {  // (d == 128: one element pair per lane)
      kv_put_i8(kv, r.seq, layer, 0, hh - n_heads, r.pos, y1, y2, lane);
    } else {
      const int kh = hh - n_heads;
      const size_t o = kv_offset(kv, r.seq, layer, 0, kh, 0, r.pos);
      kv_store(kv, o + e, y1);
      kv_store(kv, o + e + hd2, y2);
    }
  }
}

// fp32 weights: one wave per output n, all M rows; mode 0 store, 1 add, 2 swiglu
__global__ void gemv_f32_kernel(int M, int N, int K, const float* W, const float* W2, const float* x, int ldx,
                                float* out, int ldo, int mode) {
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (wave >= N) return;
  const float* w = W + (size_t)wave * K;
  const float* w2 = W2 ? W2 + (size_t)wave * K : nullptr;
  for (int m = 0; m < M; ++m) {
    const float* xr = x + (size_t)m * ldx;
    float s = 0.f, s2 = 0.f;
    for (int k = lane; k < K; k += 64) {
      s += w[k] * xr[k];
      if (mode == 2) s2 += w2[k] * xr[k];
    }
    s = wave_sum(s);
    if (mode == 2) s2 = wave_sum(s2);
    if (lane == 0) {
      float* o = out + (size_t)m * ldo + wave;
      if (mode == 0) *o = s;
      else if (mode == 1) *o += s;
      else *o = silu(s) * s2;
    }
  }
}

__global__ void argmax_rows_kernel(int N, const float* logits, int ld, int* out) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const int m = blockIdx.x;
  const float* r = logits + (size_t)m * ld;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int n = threadIdx.x; n < N; n += blockDim.x) {
    const float v = r[n];
    if (v > best || (v == best && n < bi)) { best = v; bi = n; }
  }
  wave_argmax(best, bi);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sv[w] = best; si[w] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    best = sv[0];
    bi = si[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i)
      if (sv[i] > best || (sv[i] == best && si[i] < bi)) { best = sv[i]; bi = si[i]; }
    out[m] = bi;
  }
}

__global__ void add_kernel(int n, const float* in, float* out) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) out[i] += in[i];
}

__global__ void bf16_to_f16_kernel(const uint16_t* src, _Float16* dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = (_Float16)bf16_to_f32(src[i]);
}

__global__ void f32_to_f16_kernel(const float* src, _Float16* dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = (_Float16)src[i];
}

__global__ void i8_to_f16_kernel(const int8_t* q, const uint16_t* sc, int rows, int K, _Float16* dst) {
  const size_t n = (size_t)rows * K;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = sc ? (_Float16)(bf16_to_f32(sc[i / K]) * (float)q[i]) : (_Float16)q[i];  // (sc null: the codes)
}

// dst[((rt * (K / 256) + kt) * 4 + p) * 1024 + l * 16 + 8 h + e] =
//   src[16 rt + l % 16][256 kt + 32 (2 p + h) + 8 (l / 16) + e]
__global__ void tile_i8_kernel(const int8_t* src, int8_t* dst, int N, int K) {
  const size_t n8 = (size_t)N * K / 8;  // 8-byte pieces
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n8; i += (size_t)gridDim.x * blockDim.x) {
    const int h = (int)(i & 1), l = (int)((i >> 1) & 63);
    const size_t q = i >> 7;  // (rt, kt, p)
    const int p = (int)(q & 3);
    const size_t tk = q >> 2;
    const size_t kt = tk % (K / 256), rt = tk / (K / 256);
    const size_t row = 16 * rt + (l & 15);
    const size_t col = 256 * kt + 32 * (2 * p + h) + 8 * (l >> 4);
    *(uint2*)(dst + i * 8) = *(const uint2*)(src + row * K + col);
  }
}

// dst[((rt * (K / 256) + kt) * 16 + r) * 8 + s] = src[16 rt + r][8 kt + s]
__global__ void tile_q8s_kernel(const float* src, float* dst, int N, int K) {
  const size_t n = (size_t)N * (K / 32);
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int s = (int)(i & 7), r = (int)((i >> 3) & 15);
    const size_t tk = i >> 7, kt = tk % (K / 256), rt = tk / (K / 256);
    dst[i] = src[(16 * rt + r) * (size_t)(K / 32) + 8 * kt + s];
  }
}

__global__ void tile_q40s_kernel(const uint16_t* src, uint16_t* dst, int N, int K) {
  const size_t n = (size_t)N * (K / 32);
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const int s = (int)(i & 7), r = (int)((i >> 3) & 15);
    const size_t tk = i >> 7, kt = tk % (K / 256), rt = tk / (K / 256);
    dst[i] = src[(16 * rt + r) * (size_t)(K / 32) + 8 * kt + s];  // (fp16 bits, as given)
  }
}

// one thread per output dword (lane l, k-step s of a tile and 256 columns)
__global__ void tile_q40_kernel(const uint8_t* src, uint32_t* dst, int N, int K) {
  const size_t n = (size_t)N * K / 8;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    // i = ((rt * (K / 256) + kt) * 2 + p) * 256 + l * 4 + (s % 4), s = 4 p + s % 4
    const int sl = (int)(i & 3), l = (int)((i >> 2) & 63), p = (int)((i >> 8) & 1);
    const size_t tk = i >> 9, kt = tk % (K / 256), rt = tk / (K / 256);
    const int s = 4 * p + sl;
    const size_t row = 16 * rt + (l & 15);
    const uint8_t* blk = src + row * (size_t)(K / 2) + (8 * kt + s) * 16;  // block 8 kt + s of the row
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ib = 8 * (l >> 4) + e;  // index inside the block
      const uint32_t c = ib < 16 ? (blk[ib] & 0xF) : (blk[ib - 16] >> 4);
      const int n = (e & 1) ? 4 + (e >> 1) : (e >> 1);  // nibble slot of element e
      w |= c << (4 * n);
    }
    dst[i] = w;
  }
}

// The dequantizing copies: the value (exact in fp32) rounded to fp16, or
// with lo set what that rounding left (w - fp16(w), exact in fp16 for these
// formats' few significant bits)
DPK_DEV _Float16 f16_part(float w, int lo) {
  const _Float16 h = (_Float16)w;
  return lo ? (_Float16)(w - (float)h) : h;
}

__global__ void q40_to_f16_kernel(const uint8_t* q, const uint16_t* d, int rows, int K, _Float16* dst, int lo) {
  const size_t n = (size_t)rows * K;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const size_t b = i / 32;  // block of the flat array (K % 32 == 0)
    const int ib = (int)(i & 31);
    const uint8_t byte = q[b * 16 + (ib & 15)];
    const int c = ib < 16 ? (byte & 0xF) : (byte >> 4);
    dst[i] = f16_part((float)__builtin_bit_cast(_Float16, d[b]) * (float)(c - 8), lo);
  }
}

__global__ void q8_to_f16_kernel(const int8_t* q, const float* sf, int rows, int K, _Float16* dst, int lo) {
  const size_t n = (size_t)rows * K;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = f16_part(sf[i / 32] * (float)q[i], lo);  // K % 32 == 0: block i / 32 of the flat array
}

__global__ void q4_to_f16_kernel(const uint32_t* codes, const uint16_t* sc, const uint16_t* bi, int rows, int K,
                                 _Float16* dst, int lo) {
  const size_t n = (size_t)rows * K;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / K;
    const int k = (int)(i % K);
    const uint32_t word = codes[r * (K / 8) + k / 8];
    const float c = (float)((word >> (4 * (k & 7))) & 0xF);
    const size_t g = r * (K / 64) + k / 64;
    dst[i] = f16_part(bf16_to_f32(sc[g]) * c + bf16_to_f32(bi[g]), lo);
  }
}

inline int grid_for(size_t n, int threads) {
  size_t b = (n + threads - 1) / threads;
  return (int)(b > 65536 ? 65536 : (b < 1 ? 1 : b));
}

}  // namespace

hipError_t launch_rope_table(float* cos_t, float* sin_t, int max_seq, int d, double theta, hipStream_t stream) {
  launch(rope_table_kernel, dim3(grid_for((size_t)max_seq * d / 2, 256)), dim3(256), 0, stream, cos_t,
                     sin_t, max_seq, d, theta);
  return hipGetLastError();
}

hipError_t launch_embed(int M, int H, int fmt, const void* table, const void* sc, const uint16_t* bi,
                        const RowParam* rp, const int32_t* ids_dev, int vocab, float* h, float* rs, float eps,
                        int* err_flag, hipStream_t stream, float* sq) {
  launch(embed_kernel, dim3(M), dim3(256), 0, stream, H, fmt, table, sc, bi, rp, ids_dev, vocab, h, rs,
                     eps, err_flag, sq);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_rows(int M, int H, const float* x, int ldx, const void* g, int g_is_f32, float eps,
                               void* y, int y_is_f16, int ldy, hipStream_t stream) {
  if (!g_is_f32 && g && y_is_f16 && H % 2048 == 0 && H <= 4 * 2048 && ldx % 4 == 0 && ldy % 8 == 0) {
    const uint16_t* gb = (const uint16_t*)g;
    _Float16* yb = (_Float16*)y;
    switch (H / 2048) {
      case 1: launch(rmsnorm_vec_kernel<1>, dim3(M), dim3(256), 0, stream, H, x, ldx, gb, eps, yb, y_is_f16, ldy); break;
      case 2: launch(rmsnorm_vec_kernel<2>, dim3(M), dim3(256), 0, stream, H, x, ldx, gb, eps, yb, y_is_f16, ldy); break;
      case 3: launch(rmsnorm_vec_kernel<3>, dim3(M), dim3(256), 0, stream, H, x, ldx, gb, eps, yb, y_is_f16, ldy); break;
      default: launch(rmsnorm_vec_kernel<4>, dim3(M), dim3(256), 0, stream, H, x, ldx, gb, eps, yb, y_is_f16, ldy); break;
    }
    return hipGetLastError();
  }
  launch(rmsnorm_rows_kernel, dim3(M), dim3(256), 0, stream, H, x, ldx, g, g_is_f32, eps, y, y_is_f16,
                     ldy);
  return hipGetLastError();
}

hipError_t launch_qk_rope_kv(int M, const float* qkv, int n_heads, int n_kv, int d, int qk_norm, const void* qn,
                             const void* kn, int g_is_f32, float eps, const float* rope_cos, const float* rope_sin,
                             const RowParam* rp, void* q_out, int q_is_f16, KVDesc kv, int layer,
                             hipStream_t stream) {
  if (q_is_f16 == 2 && d == 128 && !g_is_f32 && !kv.is_f32 && (qk_norm ? (qn && kn) : true)) {
    // (rows at consecutive positions of one sequence: the prefill block)
    launch(qk_rope_kv_rows_kernel, dim3((M + 63) / 64, n_heads + 2 * n_kv), dim3(256), 0, stream, qkv, M, n_heads,
           n_kv, qk_norm ? (const uint16_t*)qn : nullptr, qk_norm ? (const uint16_t*)kn : nullptr, eps, rope_cos,
           rope_sin, rp, (_Float16*)q_out, kv, layer);
    return hipGetLastError();
  }
  launch(qk_rope_kv_kernel, dim3(M, n_heads + 2 * n_kv), dim3(64), 0, stream, qkv, n_heads, n_kv, d,
                     qk_norm, qn, kn, g_is_f32, eps, rope_cos, rope_sin, rp, q_out, q_is_f16, kv, layer);
  return hipGetLastError();
}

hipError_t launch_gemv_f32(int M, int N, int K, const float* W, const float* W2, const float* x, int ldx,
                           float* out, int ldo, int mode, hipStream_t stream) {
  launch(gemv_f32_kernel, dim3((N + 3) / 4), dim3(256), 0, stream, M, N, K, W, W2, x, ldx, out, ldo,
                     mode);
  return hipGetLastError();
}

hipError_t launch_argmax_rows(int M, int N, const float* logits, int ld, int* out, hipStream_t stream) {
  launch(argmax_rows_kernel, dim3(M), dim3(1024), 0, stream, N, logits, ld, out);
  return hipGetLastError();
}

hipError_t launch_xprep(int M, int K, const float* x, int ldx, const float* sq_in, int nb, const uint16_t* g,
                        float eps, uint16_t* hi, uint16_t* lo, hipStream_t stream) {
  if (M < 1 || M > 16 || K % 32) return hipErrorInvalidValue;
  launch(xprep_kernel, dim3(M, (K + 2047) / 2048), dim3(256), 0, stream, K, x, ldx, sq_in, nb, g, eps, hi, lo);
  return hipGetLastError();
}

hipError_t launch_add(int n, const float* in, float* out, hipStream_t stream) {
  launch(add_kernel, dim3(grid_for(n, 256)), dim3(256), 0, stream, n, in, out);
  return hipGetLastError();
}

hipError_t launch_bf16_to_f16(const uint16_t* src, _Float16* dst, size_t n, hipStream_t stream) {
  launch(bf16_to_f16_kernel, dim3(grid_for(n, 256)), dim3(256), 0, stream, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_f32_to_f16(const float* src, _Float16* dst, size_t n, hipStream_t stream) {
  launch(f32_to_f16_kernel, dim3(grid_for(n, 256)), dim3(256), 0, stream, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_i8_to_f16(const int8_t* q, const uint16_t* sc, int rows, int K, _Float16* dst,
                            hipStream_t stream) {
  launch(i8_to_f16_kernel, dim3(grid_for((size_t)rows * K, 256)), dim3(256), 0, stream, q, sc, rows, K, dst);
  return hipGetLastError();
}

hipError_t launch_tile_i8(const int8_t* src, int8_t* dst, int N, int K, hipStream_t stream) {
  if (N % 16 || K % 256) return hipErrorInvalidValue;
  launch(tile_i8_kernel, dim3(grid_for((size_t)N * K / 8, 256)), dim3(256), 0, stream, src, dst, N, K);
  return hipGetLastError();
}

hipError_t launch_tile_q8s(const float* src, float* dst, int N, int K, hipStream_t stream) {
  if (N % 16 || K % 256) return hipErrorInvalidValue;
  launch(tile_q8s_kernel, dim3(grid_for((size_t)N * (K / 32), 256)), dim3(256), 0, stream, src, dst, N, K);
  return hipGetLastError();
}

hipError_t launch_tile_q40s(const uint16_t* src, uint16_t* dst, int N, int K, hipStream_t stream) {
  if (N % 16 || K % 256) return hipErrorInvalidValue;
  launch(tile_q40s_kernel, dim3(grid_for((size_t)N * (K / 32), 256)), dim3(256), 0, stream, src, dst, N, K);
  return hipGetLastError();
}

hipError_t launch_tile_q40(const uint8_t* src, uint32_t* dst, int N, int K, hipStream_t stream) {
  if (N % 16 || K % 256) return hipErrorInvalidValue;
  launch(tile_q40_kernel, dim3(grid_for((size_t)N * K / 8, 256)), dim3(256), 0, stream, src, dst, N, K);
  return hipGetLastError();
}

hipError_t launch_q40_to_f16(const uint8_t* q, const uint16_t* d, int rows, int K, _Float16* dst, hipStream_t stream,
                             bool lo) {
  launch(q40_to_f16_kernel, dim3(grid_for((size_t)rows * K, 256)), dim3(256), 0, stream, q, d, rows, K, dst, (int)lo);
  return hipGetLastError();
}

hipError_t launch_q8_to_f16(const int8_t* q, const float* sf, int rows, int K, _Float16* dst, hipStream_t stream,
                            bool lo) {
  launch(q8_to_f16_kernel, dim3(grid_for((size_t)rows * K, 256)), dim3(256), 0, stream, q, sf, rows, K, dst, (int)lo);
  return hipGetLastError();
}

hipError_t launch_q4_to_f16(const uint32_t* codes, const uint16_t* sc, const uint16_t* bi, int rows, int K,
                            _Float16* dst, hipStream_t stream, bool lo) {
  launch(q4_to_f16_kernel, dim3(grid_for((size_t)rows * K, 256)), dim3(256), 0, stream, codes, sc, bi,
                     rows, K, dst, (int)lo);
  return hipGetLastError();
}

}  // namespace dpk
