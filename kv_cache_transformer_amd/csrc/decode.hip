// K3: single-token attention over a BNSH cache (GroupQueryAttention decode,
// DecoderMaskedMultiHeadAttention self and cross attention).
//
// Work split (GroupQueryAttention page, Implementation variants: decode is
// partitioned across the key axis and partial online-softmax results are
// merged): one workgroup per (sample b, kv head, query-head group of <= 16,
// key chunk).  The workgroup streams its chunk of K/V rows once for all the
// query heads that share the kv head, so the cache is read from HBM exactly
// once per call.  A chunk's partial (max, sum, unnormalised output) goes to
// the workspace and a second kernel merges the chunks with a log-sum-exp
// combine; a sample whose keys fit one chunk is written directly.
//
// The new token's key and value are appended by the workgroup whose chunk
// holds the last row, before that workgroup reads the chunk (the key after
// the optional per-head RMSNorm and NeoX rotary; GroupQueryAttention page,
// Inputs table, q/k_norm_weight and cos/sin_cache).  The query is normed and
// rotated by every workgroup in LDS.
//
// MFMA mapping per 16-key sub-tile (wave64):
//   S^T[16 keys][16 heads] = K[16][H] . Q^T      (f16: 16x16x32, f32: 16x16x4)
//   O^T[H][16 heads]      += V^T[H][16] . P^T    (f16: 16x16x16, f32: 16x16x4)
// For f16, V^T fragments come from an identity MFMA on the row-major V
// fragment (exact: products with 1 and sums with 0), so V needs no LDS.
#include <type_traits>

#include "device_common.hpp"
#include "kvattn_internal.hpp"

namespace kvattn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kNT = 1;  // 16-key sub-tiles per wave iteration (per prefetch buffer)
// Register buffers per wave: with 3, two sub-tiles are in flight while one is
// computed; wide heads (and f32 beyond 64 dims) keep one buffer to stay
// within two waves per SIMD without spilling.
template <typename T, int HP> struct Ring { static constexpr int value = 1; };
template <> struct Ring<f16, 64> { static constexpr int value = 3; };
template <> struct Ring<f16, 128> { static constexpr int value = 3; };
template <> struct Ring<float, 64> { static constexpr int value = 3; };
constexpr int kMaxCombineChunks = 256;  // combine kernel: chunks per (sample, head)

template <typename T, int HP> struct DecTile;

// ------------------------------- f16 ----------------------------------------
// Fragments of R key/value sub-tiles are kept in registers, so that the next
// R - 1 sub-tiles' loads are in flight while one is computed.
template <int HP> struct DecTile<f16, HP> {
  static constexpr int NS = HP / 32;
  half8v qf[NS];
  float4v o[2 * NS];
  static constexpr int R = Ring<f16, HP>::value;
  half8v kf[R][kNT][NS];
  half8v vf[R][kNT][NS];

  __device__ void init() {
#pragma unroll
    for (int e = 0; e < 2 * NS; ++e) o[e] = float4v{0.f, 0.f, 0.f, 0.f};
  }
  // lane l: Q[hh = l%16][32s + 8(l/16) + i]
  __device__ void load_q(const float* qs, int sq, int lane) {
    const int hh = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[s][i] = (f16)qs[hh * sq + 32 * s + 8 * g4 + i];
  }
  // K and V rows j0 + 64u + l%16 (clamped to the last valid row), dims 32s + 8(l/16)..+7;
  // dims at or beyond H read as zero (the clamp keeps the address inside the row).
  template <int BUF>
  __device__ void load_kv(const f16* kb, const f16* vb, int j0, int last, int H, int lane) {
    const int g4 = lane >> 4;
#pragma unroll
    for (int u = 0; u < kNT; ++u) {
      const int row = min(j0 + 64 * u + (lane & 15), last);
      const f16* kr = kb + (int64_t)row * H;
      const f16* vr = vb + (int64_t)row * H;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int d = 32 * s + 8 * g4;
        const int dc = d < H ? d : 0;
        half8v k = load_half8(kr + dc), v = load_half8(vr + dc);
        if (d >= H) { k = half8v{}; v = half8v{}; }
        kf[BUF][u][s] = k;
        vf[BUF][u][s] = v;
      }
    }
  }
  // sc[u][i] = S^T[key j0 + 64u + 4(l/16) + i][head l%16]
  template <int BUF>
  __device__ void scores(float4v (&sc)[kNT]) {
#pragma unroll
    for (int u = 0; u < kNT; ++u) {
      float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) acc = mfma16x16x32(kf[BUF][u][s], qf[s], acc);
      sc[u] = acc;
    }
  }
  __device__ void scale_o(float a) {
#pragma unroll
    for (int e = 0; e < 2 * NS; ++e) o[e] *= a;
  }
  template <int BUF>
  __device__ void pv(const float4v (&p)[kNT], half4v ident) {
    const float4v zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kNT; ++u) {
      half4v pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = (f16)p[u][i];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const half8v v = vf[BUF][u][s];
        const float4v tl = mfma16x16x16(half4v{v[0], v[1], v[2], v[3]}, ident, zero);
        const float4v th = mfma16x16x16(half4v{v[4], v[5], v[6], v[7]}, ident, zero);
        half4v al, ah;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          al[i] = (f16)tl[i];
          ah[i] = (f16)th[i];
        }
        o[2 * s] = mfma16x16x16(al, pb, o[2 * s]);
        o[2 * s + 1] = mfma16x16x16(ah, pb, o[2 * s + 1]);
      }
    }
  }
  // lane l holds O^T[32s + 8(l/16) + 4*half + i][head l%16]
  __device__ void store_o(float* so, int sq, int lane) {
    const int hh = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int i = 0; i < 4; ++i) so[hh * sq + 32 * s + 8 * g4 + 4 * hf + i] = o[2 * s + hf][i];
  }
};

// ------------------------------- f32 ----------------------------------------
template <int HP> struct DecTile<float, HP> {
  static constexpr int NU = HP / 16;
  float qf[NU][4];
  float4v o[NU];
  static constexpr int R = Ring<float, HP>::value;
  float4v kf[R][kNT][NU];
  float vf[R][kNT][4][NU];

  __device__ void init() {
#pragma unroll
    for (int t = 0; t < NU; ++t) o[t] = float4v{0.f, 0.f, 0.f, 0.f};
  }
  // lane l: Q[hh = l%16][16t + 4(l/16) + e]
  __device__ void load_q(const float* qs, int sq, int lane) {
    const int hh = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int t = 0; t < NU; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[t][e] = qs[hh * sq + 16 * t + 4 * g4 + e];
  }
  template <int BUF>
  __device__ void load_kv(const float* kb, const float* vb, int j0, int last, int H, int lane) {
    const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int u = 0; u < kNT; ++u) {
      const int krow = min(j0 + 64 * u + l16, last);
      const float* kr = kb + (int64_t)krow * H;
#pragma unroll
      for (int t = 0; t < NU; ++t) {
        const int d = 16 * t + 4 * g4;
        float4v k = *reinterpret_cast<const float4v*>(kr + (d < H ? d : 0));
        kf[BUF][u][t] = (d < H) ? k : float4v{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int vrow = min(j0 + 64 * u + 4 * g4 + k, last);
        const float* vr = vb + (int64_t)vrow * H;
#pragma unroll
        for (int t = 0; t < NU; ++t) {
          const int d = 16 * t + l16;
          const float v = vr[d < H ? d : 0];
          vf[BUF][u][k][t] = (d < H) ? v : 0.f;
        }
      }
    }
  }
  template <int BUF>
  __device__ void scores(float4v (&sc)[kNT]) {
#pragma unroll
    for (int u = 0; u < kNT; ++u) {
      float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < NU; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma16x16x4f32(kf[BUF][u][t][e], qf[t][e], acc);
      sc[u] = acc;
    }
  }
  __device__ void scale_o(float a) {
#pragma unroll
    for (int t = 0; t < NU; ++t) o[t] *= a;
  }
  template <int BUF>
  __device__ void pv(const float4v (&p)[kNT], half4v) {
#pragma unroll
    for (int u = 0; u < kNT; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int t = 0; t < NU; ++t) o[t] = mfma16x16x4f32(vf[BUF][u][k][t], p[u][k], o[t]);
  }
  // lane l holds O^T[16t + 4(l/16) + i][head l%16]
  __device__ void store_o(float* so, int sq, int lane) {
    const int hh = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int t = 0; t < NU; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) so[hh * sq + 16 * t + 4 * g4 + i] = o[t][i];
  }
};

// Key count n and the row of the appended token (-1: none) for sample b.
__device__ __forceinline__ void decode_len(const DecodeParams& p, int b, int& n, int& newrow) {
  if (p.len_mode == 0) n = p.lens[b] + 1;
  else if (p.len_mode == 1) n = p.lens[0] + 1;
  else n = p.host_n;
  newrow = (p.k_new != nullptr) ? n - 1 : -1;
  if (n > p.cap) { n = p.cap; newrow = -1; }  // precondition violated: stay in bounds
  if (n < 0) { n = 0; newrow = -1; }
}

__device__ __forceinline__ int decode_kstart(const DecodeParams& p, int n) {
  return (p.window >= 0) ? max(0, n - 1 - p.window) : 0;
}

// Chunks of this sample, at least one (it writes the output even with no
// keys) and at most the grid's max_chunks (lengths beyond the host's total
// are a violated precondition; the extra keys are then not read).
__device__ __forceinline__ int decode_nchunks(const DecodeParams& p, int n, int kstart) {
  return min(max(1, (n - kstart + p.chunk - 1) / p.chunk), p.max_chunks);
}

template <typename T>
__device__ __forceinline__ float read_sink(const DecodeParams& p, int h, bool& has) {
  if (p.sink != nullptr) {
    has = true;
    return kLog2e * to_f32(static_cast<const T*>(p.sink)[h]);
  }
  has = (p.smooth == 1);
  return 0.f;
}

// FEAT bits: kSoftcap (scores are soft-capped), kExtras (additive bias and/or
// mask, and/or the qk output).  The plain variant has no per-score checks.
constexpr int kSoftcap = 1, kExtras = 2;

template <typename T, int HP, int FEAT>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(DecodeParams p) {
  __shared__ float smem[kWaves * 16 * (HP + 4)];
  __shared__ float s_m[kWaves][16], s_l[kWaves][16], s_r[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x;
  const int kvh = blockIdx.y / p.head_groups;
  const int hgrp = blockIdx.y % p.head_groups;
  const int b = blockIdx.z;
  const int H = p.H;
  const int g = p.N / p.kvN;
  const int h0 = kvh * g + hgrp * 16;
  const int nh = min(16, g - hgrp * 16);

  int n, newrow;
  decode_len(p, b, n, newrow);
  const int kstart = decode_kstart(p, n);
  const int nchunks = decode_nchunks(p, n, kstart);
  if (c >= nchunks) return;
  const int c0 = kstart + c * p.chunk;
  const int c1 = min(c0 + p.chunk, n);

  const T* qg = static_cast<const T*>(p.q) + (int64_t)b * p.N * H;
  T* kb = static_cast<T*>(p.kc) + ((int64_t)b * p.kvN + kvh) * p.cap * H;
  T* vb = static_cast<T*>(p.vc) + ((int64_t)b * p.kvN + kvh) * p.cap * H;
  const int half = H / 2;
  const T* cs = static_cast<const T*>(p.cos);
  const T* sn = static_cast<const T*>(p.sin);

  // ---- append the new token's key/value (the workgroup whose chunk holds its
  // row does it before it reads any key row, so that its loads see the row) --
  if (newrow >= 0 && newrow >= c0 && newrow < c1) {
    const T* kn = static_cast<const T*>(p.k_new) + ((int64_t)b * p.kvN + kvh) * H;
    const T* vn = static_cast<const T*>(p.v_new) + ((int64_t)b * p.kvN + kvh) * H;
    if (wave == 0) {
      float rinv = 1.f;
      if (p.k_norm != nullptr) {
        float ss = 0.f;
        for (int d = lane; d < H; d += 64) { float x = to_f32(kn[d]); ss += x * x; }
        ss = wave_sum_xor(ss, 1, 32);
        rinv = rsqrtf(ss / (float)H + p.eps);
      }
      const T* kw = static_cast<const T*>(p.k_norm);
      for (int i = lane; i < half; i += 64) {
        float a = to_f32(kn[i]), e = to_f32(kn[i + half]);
        if (kw != nullptr) {
          a *= rinv * to_f32(kw[i]);
          e *= rinv * to_f32(kw[i + half]);
        }
        if (cs != nullptr) {
          const int rrow = min(newrow, p.rot_rows - 1);
          const float co = to_f32(cs[(int64_t)rrow * half + i]);
          const float si = to_f32(sn[(int64_t)rrow * half + i]);
          const float a2 = a * co - e * si;
          const float e2 = e * co + a * si;
          a = a2;
          e = e2;
        }
        kb[(int64_t)newrow * H + i] = from_f32<T>(a);
        kb[(int64_t)newrow * H + i + half] = from_f32<T>(e);
      }
    } else if (wave == 1) {
      for (int d = lane; d < H; d += 64) vb[(int64_t)newrow * H + d] = vn[d];
    }
    __syncthreads();
  }

  // ---- start streaming: the first R - 1 sub-tiles' loads go out now, so the
  // query set-up below overlaps with them --------------------------------------
  DecTile<T, HP> tile;
  tile.init();
  constexpr int R = DecTile<T, HP>::R;
  const int step = 16 * kWaves * kNT;
  const int first = c0 + 16 * wave;
  const int nsub = first < c1 ? (c1 - first + step - 1) / step : 0;
  auto jof = [&](int k) { return first + k * step; };
  if constexpr (R == 3) {
    if (nsub > 0) tile.template load_kv<0>(kb, vb, jof(0), c1 - 1, H, lane);
    if (nsub > 1) tile.template load_kv<1>(kb, vb, jof(1), c1 - 1, H, lane);
  }

  // ---- query heads into LDS (float), per-head RMSNorm and rotary ------------
  // The rotary table entries of this thread's pairs are loaded together with
  // the query so that the set-up waits for memory once.
  constexpr int SQ = HP + 4;                    // padded LDS row (floats)
  constexpr int PH = HP / 2;                    // rotary pairs per padded head
  constexpr int PPT = 16 * PH / kThreads;       // pairs per thread
  float* qs = smem;
  for (int idx = tid; idx < 16 * HP; idx += kThreads) {
    const int hh = idx / HP, d = idx % HP;
    qs[hh * SQ + d] = (hh < nh && d < H) ? to_f32(qg[(h0 + hh) * H + d]) : 0.f;
  }
  const int pos = min(max(n - 1, 0), max(p.rot_rows - 1, 0));
  float co_r[PPT], si_r[PPT];
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int i = (tid + kThreads * k) % PH;
    co_r[k] = (cs != nullptr && i < half) ? to_f32(cs[(int64_t)pos * half + i]) : 1.f;
    si_r[k] = (cs != nullptr && i < half) ? to_f32(sn[(int64_t)pos * half + i]) : 0.f;
  }
  __syncthreads();
  if (p.q_norm != nullptr) {
    // 16 lanes per head
    const int hh = tid >> 4, part = tid & 15;
    float ss = 0.f;
    for (int d = part; d < H; d += 16) ss += qs[hh * SQ + d] * qs[hh * SQ + d];
    ss = wave_sum_xor(ss, 1, 8);
    if (part == 0) s_r[hh] = rsqrtf(ss / (float)H + p.eps);
    __syncthreads();
  }
  if (p.q_norm != nullptr || cs != nullptr) {
    const T* qw = static_cast<const T*>(p.q_norm);
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int idx = tid + kThreads * k;
      const int hh = idx / PH, i = idx % PH;
      if (hh < nh && i < half) {
        float a = qs[hh * SQ + i], e = qs[hh * SQ + i + half];
        if (qw != nullptr) {
          a *= s_r[hh] * to_f32(qw[i]);
          e *= s_r[hh] * to_f32(qw[i + half]);
        }
        const float a2 = a * co_r[k] - e * si_r[k];
        const float e2 = e * co_r[k] + a * si_r[k];
        qs[hh * SQ + i] = a2;
        qs[hh * SQ + i + half] = e2;
      }
    }
    __syncthreads();
  }
  tile.load_q(qs, SQ, lane);
  __syncthreads();  // qs is reused below

  // identity for the f16 V transpose: lane l holds B[k = 4(l/16)+i][n = l%16]
  half4v ident;
#pragma unroll
  for (int i = 0; i < 4; ++i) ident[i] = (f16)((4 * (lane >> 4) + i) == (lane & 15) ? 1.f : 0.f);

  const int hh = lane & 15;
  const bool head_ok = hh < nh;
  const int h = h0 + hh;
  const float scale = p.scale;
  const float cap = p.softcap, inv_cap = p.softcap > 0.f ? 1.f / p.softcap : 0.f;
  const T* bias = static_cast<const T*>(p.bias);
  T* qk = static_cast<T*>(p.qk);

  float m = kNegInf, l = 0.f;
  // Score transform, online softmax and PV for the sub-tiles held in BUF.
  auto process = [&](auto buf_tag, int j0) {
    constexpr int BUF = decltype(buf_tag)::value;
    float4v sc[kNT];
    tile.template scores<BUF>(sc);
    mfma_result_fence();
    float tmax = kNegInf;
    float4v x[kNT];
#pragma unroll
    for (int u = 0; u < kNT; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = j0 + 64 * u + 4 * (lane >> 4) + i;
        const bool ok = head_ok && key < c1;
        float v = sc[u][i] * scale;
        if (FEAT & kSoftcap) v = softcap_apply(v, cap, inv_cap);
        if (FEAT & kExtras) {
          if (ok && bias != nullptr && key < p.bias_cols)
            v += to_f32(bias[b * p.bias_sb + h * p.bias_sh + key]);
          if (ok && p.mask != nullptr && key < p.mask_cols)
            v += (p.mask[(int64_t)b * p.mask_cols + key] == 0) ? p.mask_filter : 0.f;
          if (ok && qk != nullptr) qk[((int64_t)b * p.N + h) * p.host_n + key] = from_f32<T>(v);
        }
        v = ok ? v * kLog2e : kNegInf;
        x[u][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const float mnew = fmaxf(m, tmax);
    const float muse = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = fast_exp2(m - muse);
    m = mnew;
    float4v pr[kNT];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < kNT; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = fast_exp2(x[u][i] - muse);
        pr[u][i] = e;
        psum += e;
      }
    l = l * alpha + psum;
    tile.scale_o(alpha);
    tile.template pv<BUF>(pr, ident);
  };

  // Each wave walks its sub-tiles (every kWaves-th one of the chunk) through a
  // ring of R register buffers, loads running R - 1 sub-tiles ahead (the
  // first R - 1 were issued before the query set-up).
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if constexpr (R == 3) {
    for (int k = 0; k < nsub; k += 3) {
      if (k + 2 < nsub) tile.template load_kv<2>(kb, vb, jof(k + 2), c1 - 1, H, lane);
      process(I0{}, jof(k));
      if (k + 1 >= nsub) break;
      if (k + 3 < nsub) tile.template load_kv<0>(kb, vb, jof(k + 3), c1 - 1, H, lane);
      process(I1{}, jof(k + 1));
      if (k + 2 >= nsub) break;
      if (k + 4 < nsub) tile.template load_kv<1>(kb, vb, jof(k + 4), c1 - 1, H, lane);
      process(I2{}, jof(k + 2));
    }
  } else {
    static_assert(R == 1, "ring depth 1 or 3");
    for (int k = 0; k < nsub; ++k) {
      tile.template load_kv<0>(kb, vb, jof(k), c1 - 1, H, lane);
      process(I0{}, jof(k));
    }
  }
  mfma_result_fence();
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);

  // ---- merge the waves of this workgroup ------------------------------------
  float* so = smem + wave * 16 * SQ;
  tile.store_o(so, SQ, lane);
  if (lane < 16) {
    s_m[wave][lane] = m;
    s_l[wave][lane] = l;
  }
  __syncthreads();

  const int rec = HP + 2;
  for (int idx = tid; idx < nh * H; idx += kThreads) {
    const int hj = idx / H, d = idx % H;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][hj]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      float f = fast_exp2(s_m[w][hj] - Mu);
      L += s_l[w][hj] * f;
      O += smem[w * 16 * SQ + hj * SQ + d] * f;
    }
    const int hq = h0 + hj;
    if (nchunks == 1) {
      bool has;
      float sg = read_sink<T>(p, hq, has);
      float out;
      if (has) {
        float M2 = fmaxf(M, sg);
        float den = L * fast_exp2(M - M2) + fast_exp2(sg - M2);
        out = O * fast_exp2(M - M2) / den;
        if (L == 0.f) out = 0.f;
      } else {
        out = (L > 0.f) ? O / L : 0.f;
      }
      static_cast<T*>(p.out)[((int64_t)b * p.N + hq) * H + d] = from_f32<T>(out);
    } else {
      float* rp = p.part + (((int64_t)b * p.N + hq) * p.max_chunks + c) * rec;
      if (d == 0) {
        rp[0] = M;
        rp[1] = L;
      }
      rp[2 + d] = O;
    }
  }
}

// Merge the chunk partials of one (sample, query head): the chunk maxima and
// sums are read by all threads at once into LDS, then every thread sums its
// dims over the chunks with independent loads.
template <typename T, int HP>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
  __shared__ float w_s[kMaxCombineChunks];
  __shared__ float red[2][4];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int n, newrow;
  decode_len(p, b, n, newrow);
  const int kstart = decode_kstart(p, n);
  const int nchunks = decode_nchunks(p, n, kstart);
  if (nchunks <= 1) return;
  const int rec = HP + 2;
  const float* base = p.part + ((int64_t)b * p.N + h) * p.max_chunks * rec;
  // chunk maxima -> weights exp2(M_c - M), and the weighted sum of the L_c
  float mc = kNegInf, lc = 0.f;
  if (tid < nchunks) {
    mc = base[tid * rec];
    lc = base[tid * rec + 1];
  }
  const int wave = tid >> 6, nw = blockDim.x >> 6;
  float M = wave_max_xor(mc, 1, 32);
  if ((tid & 63) == 0) red[0][wave] = M;
  __syncthreads();
  M = red[0][0];
  for (int w = 1; w < nw; ++w) M = fmaxf(M, red[0][w]);
  const float Mu = (M == kNegInf) ? 0.f : M;
  const float wgt = (tid < nchunks) ? fast_exp2(mc - Mu) : 0.f;
  if (tid < nchunks) w_s[tid] = wgt;
  float L = wave_sum_xor(lc * wgt, 1, 32);
  if ((tid & 63) == 0) red[1][wave] = L;
  __syncthreads();
  L = red[1][0];
  for (int w = 1; w < nw; ++w) L += red[1][w];
  bool has;
  const float sg = read_sink<T>(p, h, has);
  float inv;
  if (L == 0.f) {
    inv = 0.f;
  } else if (has) {
    const float M2 = fmaxf(M, sg);
    const float den = L * fast_exp2(M - M2) + fast_exp2(sg - M2);
    inv = fast_exp2(M - M2) / den;
  } else {
    inv = 1.f / L;
  }
  for (int d = tid; d < p.H; d += blockDim.x) {
    float O = 0.f;
#pragma unroll 8
    for (int c = 0; c < nchunks; ++c) O += base[c * rec + 2 + d] * w_s[c];
    static_cast<T*>(p.out)[((int64_t)b * p.N + h) * p.H + d] = from_f32<T>(O * inv);
  }
}

template <typename T, int HP, int FEAT>
hipError_t launch_decode_f(const DecodeParams& p, hipStream_t s) {
  dim3 grid(p.max_chunks, p.kvN * p.head_groups, p.B);
  hipLaunchKernelGGL((decode_kernel<T, HP, FEAT>), grid, dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_chunks <= 1) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, HP>), dim3(p.N, p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename T, int HP>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
  const bool extras = p.bias != nullptr || p.mask != nullptr || p.qk != nullptr;
  const bool cap = p.softcap > 0.f;
  if (extras) {
    if (cap) return launch_decode_f<T, HP, kSoftcap | kExtras>(p, s);
    return launch_decode_f<T, HP, kExtras>(p, s);
  }
  if (cap) return launch_decode_f<T, HP, kSoftcap>(p, s);
  return launch_decode_f<T, HP, 0>(p, s);
}

}  // namespace

hipError_t launch_decode(DType dt, int hp, const DecodeParams& p, hipStream_t s) {
  if (dt == DType::F16) {
    if (hp == 64) return launch_decode_t<f16, 64>(p, s);
    if (hp == 128) return launch_decode_t<f16, 128>(p, s);
    return launch_decode_t<f16, 256>(p, s);
  }
  if (hp == 64) return launch_decode_t<float, 64>(p, s);
  if (hp == 128) return launch_decode_t<float, 128>(p, s);
  return launch_decode_t<float, 256>(p, s);
}

}  // namespace kvattn
