// Prefill attention on gfx950 matrix cores: causal grouped-query attention of
// M query rows (positions start..start+M-1) over the cached keys 0..pos of one
// sequence, softmax(q k^T / sqrt(d)) v per head ("LLMs on the ANE", "What's
// inside": decomposed causal attention; KV head h / G serves query head h).
//
// Formulated transposed so that every softmax statistic is lane-local:
//   S^T = K Q^T      (A = K tile rows = keys, B = Q^T columns = queries)
//   O^T += V^T P^T   (A = V^T tile rows = channels, B = P^T)
// With v_mfma_f32_32x32x16_f16 a lane owns one query column, so the running
// max / sum / rescale of the online softmax need one cross-lane step (the
// partner half-wave).  The accumulator layout of S^T is reused directly as the
// B operand of the second product by permuting the key order inside each
// 16-key step; the V^T tile is read from LDS with the same permutation.
//
// Precision: q, P and the output are each carried as fp16 hi + lo parts
// (two MFMAs per product), so the only 16-bit rounding left is that of the
// cached K and V.
//
// int8 cache (KV8): the tiles are staged as fp16 s * q, s the position's scale
// (one more fp16 rounding, of the same size as the fp16 cache's own).
//
// Workgroup: 4 waves, each one query head x 32 query rows; the heads of a
// workgroup share one KV head, so each K / V^T tile (64 keys) is staged in LDS
// once for all of them.
#include "common.h"
#include "kernels.h"

namespace dpk {

namespace {

constexpr int THREADS = 256;
constexpr int BKV = 64;
constexpr int D = 128;
constexpr int KSTR = D + 8;     // halfs per K row in LDS
constexpr int VSTR = BKV + 8;   // halfs per V^T row in LDS
constexpr float LOG2E = 1.4426950408889634f;

// (int8 cache: one workgroup per CU -- the staging registers of the codes and
// scales do not fit beside the fp16 kernel's 254 at two)
template <bool KV8>
__global__ __launch_bounds__(THREADS, KV8 ? 1 : 2) void attn_prefill_kernel(AttnPrefillArgs a, int heads_per_wg, int rb_per_wg,
                                                                    int n_rb, int n_hg) {
  __shared__ __attribute__((aligned(16))) _Float16 Ks[BKV][KSTR];
  __shared__ __attribute__((aligned(16))) _Float16 Vs[D][VSTR];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int G = a.n_heads / a.n_kv;
  // (row block, head group) items in order of causal length, longest first:
  // the first half of the grid takes them from the longest end, the second
  // half from the shortest end, so a compute unit holding workgroups L and
  // L + half pairs a long item with a short one instead of two of equal length
  const int total = n_rb * n_hg, half = (total + 1) / 2, L = (int)blockIdx.x;
  const int k = L < half ? L : total - 1 - (L - half);
  const int rbw = n_rb - 1 - k / n_hg;
  const int head0 = (k % n_hg) * heads_per_wg;
  const int g = head0 / G;
  const int head = head0 + wave % heads_per_wg;
  const int r0 = (rbw * rb_per_wg + wave / heads_per_wg) * 32;  // this wave's first query row
  const int wg_r1 = min(a.M, (rbw + 1) * rb_per_wg * 32);         // workgroup's last row + 1
  const int q32 = lane & 31, hh = lane >> 5;
  const int qrow = r0 + q32;
  const bool row_ok = qrow < a.M;
  const int qpos = a.start + (row_ok ? qrow : a.M - 1);
  const float c = a.scale * LOG2E;

  // Q^T fragments: lane (query q32, k-group hh) holds q[16 s + 8 hh .. +7],
  // as fp16 hi and lo parts (q = hi + lo to ~22 bits)
  f16x8 qf[D / 16], qlo[D / 16];
  {
    const _Float16* qp = a.q + ((size_t)(row_ok ? qrow : a.M - 1) * a.n_heads + head) * D;
    const _Float16* qlp = qp + (size_t)a.M * a.n_heads * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qf[s] = *(const f16x8*)(qp + 16 * s + 8 * hh);
      qlo[s] = *(const f16x8*)(qlp + 16 * s + 8 * hh);
    }
    // fold the softmax scale (and log2 e) into q once: q c split again
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = ((float)qf[s][e] + (float)qlo[s][e]) * c;
        const _Float16 h = (_Float16)x;
        qf[s][e] = h;
        qlo[s][e] = (_Float16)(x - (float)h);
      }
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[i][v] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;

  const _Float16* Kg = (const _Float16*)a.kv.base + kv_slab(a.kv, a.seq, a.layer, 0, g);
  const _Float16* Vg = (const _Float16*)a.kv.base + kv_slab(a.kv, a.seq, a.layer, 1, g);
  const int kend = a.start + wg_r1;  // keys [0, kend) are visible to some row here
  const int wave_kend = a.start + min(a.M, r0 + 32);
  // K [64 keys][128] and V^T [128][64 keys] of a tile: global -> registers
  // one tile ahead (the loads fly while the current tile is computed), then
  // registers -> LDS.  The V^T row stride (kv.max_seq) is a multiple of 64, so
  // an 8-key load stays inside the row.
  u32x4 kreg[4];
  f16x8 vreg[4];
  // int8 cache: codes (8 per piece) and the scales of their key(s)
  const int8_t* K8 = (const int8_t*)a.kv.base + kv_slab(a.kv, a.seq, a.layer, 0, g);
  const int8_t* V8 = (const int8_t*)a.kv.base + kv_slab(a.kv, a.seq, a.layer, 1, g);
  const float* Ksc = KV8 ? a.kv.scales + kv_scale_slab(a.kv, a.seq, a.layer, 0, g) : nullptr;
  const float* Vsc = KV8 ? a.kv.scales + kv_scale_slab(a.kv, a.seq, a.layer, 1, g) : nullptr;
  // (a thread's V pieces share their 8 keys: idx & 7 == tid & 7)
  u32x2 kq[4], vq[4];
  float ksf[4];
  f32x4 vsf[2];
  auto gload = [&](int k0) {
    const bool tail = k0 + BKV > kend;  // uniform: only the last tile has keys past kend
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + THREADS * i;  // 0..1023
      const int kr = idx >> 4, kc = (idx & 15) * 8;
      const int krow = tail ? min(k0 + kr, kend - 1) : k0 + kr;
      const int vr = idx >> 3, vc = (idx & 7) * 8;
      if constexpr (KV8) {
        kq[i] = *(const u32x2*)(K8 + (size_t)krow * D + kc);
        ksf[i] = Ksc[krow];
        vq[i] = *(const u32x2*)(V8 + (size_t)vr * a.kv.max_seq + k0 + vc);
        if (i == 0) {
          vsf[0] = *(const f32x4*)(Vsc + k0 + vc);
          vsf[1] = *(const f32x4*)(Vsc + k0 + vc + 4);
        }
      } else {
        kreg[i] = *(const u32x4*)(Kg + (size_t)krow * D + kc);
        vreg[i] = *(const f16x8*)(Vg + (size_t)vr * a.kv.max_seq + k0 + vc);
      }
    }
  };
  auto lstore = [&](int k0) {
    const bool tail = k0 + BKV > kend;  // uniform over the workgroup
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + THREADS * i;
      const int kr = idx >> 4, kc = (idx & 15) * 8;
      const int vr = idx >> 3, vc = (idx & 7) * 8;
      if constexpr (KV8) {  // s * q as fp16
        f16x8 kk, v8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t kw = e < 4 ? kq[i].x : kq[i].y, vw = e < 4 ? vq[i].x : vq[i].y;
          kk[e] = (_Float16)(ksf[i] * (float)(int8_t)(kw >> (8 * (e & 3))));
          v8[e] = (_Float16)(vsf[e >> 2][e & 3] * (float)(int8_t)(vw >> (8 * (e & 3))));
        }
        kreg[i] = __builtin_bit_cast(u32x4, kk);
        vreg[i] = v8;
      }
      *(u32x4*)&Ks[kr][kc] = kreg[i];
      // keys at or past kend are zeroed (the cache there may hold any bit
      // pattern, and 0 * NaN would poison O); only the last tile has any
      f16x8 vv = vreg[i];
      if (tail) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (k0 + vc + e >= kend) vv[e] = (_Float16)0.f;
      }
      *(f16x8*)&Vs[vr][vc] = vv;
    }
  };
  gload(0);
  for (int k0 = 0; k0 < kend; k0 += BKV) {
    __syncthreads();  // the previous tile's LDS reads are done (and this tile's loads have landed)
    lstore(k0);
    __syncthreads();
    if (k0 + BKV < kend) gload(k0 + BKV);
    if (k0 >= wave_kend) continue;  // every key of this tile is after this wave's rows
    // S^T for two blocks of 32 keys
    f32x16 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[b][v] = 0.f;
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const f16x8 kf = *(const f16x8*)&Ks[b * 32 + q32][16 * st + 8 * hh];
        s[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[st], s[b], 0, 0, 0);
        s[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qlo[st], s[b], 0, 0, 0);
      }
    }
    // mask + online softmax (log2 domain; q carries the scale); lane key
    // index = 8(v/4) + 4hh + v%4.  Only tiles that reach past this wave's
    // first row (the diagonal) or past kend need the mask.
    float tmax = -INFINITY;
    if (k0 + BKV - 1 > a.start + r0 || k0 + BKV > kend) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = k0 + b * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
          if (key > qpos || key >= kend) s[b][v] = -INFINITY;
          tmax = fmaxf(tmax, s[b][v]);
        }
    } else {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, s[b][v]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mnew = fmaxf(mrun, tmax);
    const float alpha = (mrun == -INFINITY) ? 0.f : exp2f(mrun - mnew);
    float psum = 0.f;
    f16x8 pf[2][2], pl[2][2];  // P as fp16 hi + lo
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        // mnew is finite (key 0 is visible to every row, and the first tile
        // a wave computes is k0 = 0), so a masked -inf gives exactly 0; the
        // hardware exp2 (results below 2^-126 flush to 0, immaterial here)
        const float p0 = __builtin_amdgcn_exp2f(s[b][v] - mnew), p1 = __builtin_amdgcn_exp2f(s[b][v + 1] - mnew);
        psum += p0 + p1;
        // hi: two at once, rounded toward zero (lo = p - hi takes the rest, so
        // hi + lo keeps ~22 bits either way)
        const auto h2 = __builtin_amdgcn_cvt_pkrtz(p0, p1);
        const auto l2 = __builtin_amdgcn_cvt_pkrtz(p0 - (float)h2[0], p1 - (float)h2[1]);
        pf[b][v >> 3][v & 7] = h2[0];
        pf[b][v >> 3][(v & 7) + 1] = h2[1];
        pl[b][v >> 3][v & 7] = l2[0];
        pl[b][v >> 3][(v & 7) + 1] = l2[1];
      }
    psum += __shfl_xor(psum, 32, 64);
    lrun = lrun * alpha + psum;
    // O only needs rescaling when some query's running maximum moved (alpha
    // is exactly 1 otherwise); past the first tiles that is rare
    const bool moved = __builtin_amdgcn_ballot_w64(mnew != mrun) != 0;
    mrun = mnew;
    if (moved) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] *= alpha;
    }
    // O^T += V^T P^T; key slots of k-group hh in step (b, t):
    //   b*32 + 16t + {4hh..4hh+3, 8+4hh..8+4hh+3}
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int kb = b * 32 + 16 * t + 4 * hh;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
          const int dr = i * 32 + q32;
          const u32x2 lo = *(const u32x2*)&Vs[dr][kb];
          const u32x2 hi = *(const u32x2*)&Vs[dr][kb + 8];
          const u32x4 vw = {lo.x, lo.y, hi.x, hi.y};
          const f16x8 vf = __builtin_bit_cast(f16x8, vw);
          o[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[b][t], o[i], 0, 0, 0);
          o[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pl[b][t], o[i], 0, 0, 0);
        }
      }
  }
  if (!row_ok) return;
  const float inv = 1.0f / lrun;
  // row layout [hi: n_heads * D][lo: n_heads * D]
  _Float16* op = a.out + (size_t)qrow * 2 * a.n_heads * D + (size_t)head * D;
  _Float16* olp = op + (size_t)a.n_heads * D;
  // O^T block i: channel = 32 i + 8 (v/4) + 4 hh + v%4 for query q32
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      f16x4 w, wl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = o[i][4 * v4 + e] * inv;
        w[e] = (_Float16)x;
        wl[e] = (_Float16)(x - (float)w[e]);
      }
      *(f16x4*)(op + 32 * i + 8 * v4 + 4 * hh) = w;
      *(f16x4*)(olp + 32 * i + 8 * v4 + 4 * hh) = wl;
    }
}

}  // namespace

hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t stream) {
  if (a.d != D || a.kv.is_f32 || a.kv.max_seq % BKV) return hipErrorInvalidValue;
  const int G = a.n_heads / a.n_kv;
  const int hpw = G < 4 ? G : 4;
  if (G % hpw || 4 % hpw) return hipErrorInvalidValue;
  const int rbpw = 4 / hpw;
  const int n_rb = (a.M + 32 * rbpw - 1) / (32 * rbpw);
  const int n_hg = a.n_heads / hpw;
  if (a.kv.i8)
    launch(attn_prefill_kernel<true>, dim3(n_rb * n_hg), dim3(THREADS), 0, stream, a, hpw, rbpw, n_rb, n_hg);
  else
    launch(attn_prefill_kernel<false>, dim3(n_rb * n_hg), dim3(THREADS), 0, stream, a, hpw, rbpw, n_rb, n_hg);
  return hipGetLastError();
}

}  // namespace dpk
