// K3: single-token attention over a BNSH cache (GroupQueryAttention decode,
// DecoderMaskedMultiHeadAttention self and cross attention).
//
// Work split (GroupQueryAttention page, Implementation variants: decode is
// partitioned along the key axis and the partial online-softmax results are
// merged).  A unit is (sample b, kv head, group of <= 16 query heads sharing
// that kv head).  Every wave of the grid is an independent worker: the live
// keys of all units are dealt out so that each wave streams about the same
// number of key rows, each unit receiving a whole number of waves (at least
// one) and each of its waves one contiguous run of its keys.  The lengths are
// device data, so every wave derives the deal from them itself.  A wave reads
// its rows of the cache once for all query heads of its unit, with up to
// three 16-row sub-tiles in flight in a register ring, and writes one partial
// (max, sum, unnormalised output) per head; a unit served by a single wave
// writes the output directly.  decode_combine_kernel merges the partials with
// a log-sum-exp combine and adds the head-sink term.
//
// The query (optionally RMS-normed per head, then NeoX-rotated at the new
// token's position) is built in registers in the MFMA operand layout; its
// loads are issued before the first key/value loads so that waiting for it
// does not wait for them.  The new token's key (normed and rotated the same
// way) and value are appended by the wave whose run holds the new row, before
// that wave loads the row (GroupQueryAttention page, Inputs table:
// past_key/present_key, q/k_norm_weight, cos/sin_cache).  Lanes of one wave
// see each other's global stores in program order, so no barrier is needed.
//
// MFMA mapping per 16-key sub-tile (wave64):
//   S^T[16 keys][16 heads] = K[16][H] . Q^T      (f16: 16x16x32, f32: 16x16x4)
//   O^T[H][16 heads]      += V^T[H][16] . P^T    (f16: 16x16x16, f32: 16x16x4)
// For f16 the V^T fragments come from an identity MFMA on the row-major V
// fragment (exact: products with 1 and sums with 0), so V needs no LDS.
#include <type_traits>
#include <utility>

#include "device_common.hpp"
#include "kvattn_internal.hpp"

namespace kvattn {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerGroup = kThreads / 64;
constexpr int64_t kMinKeysPerWave = 64;

// Register ring depth (16-row sub-tiles held per wave): R - 1 are in flight
// while one is computed.  Sized to stay within 256 registers per lane (two
// waves per SIMD) without spilling.
template <typename T, int HP> struct Ring { static constexpr int value = 1; };
template <> struct Ring<f16, 64> { static constexpr int value = 4; };
template <> struct Ring<f16, 128> { static constexpr int value = 4; };
template <> struct Ring<float, 64> { static constexpr int value = 3; };
template <> struct Ring<float, 128> { static constexpr int value = 2; };

// Four consecutive elements of a head row ("quad"): the unit of the query
// set-up, the append and the output stores.
template <typename T> struct Quad;
template <> struct Quad<f16> {
  using type = half4v;
  __device__ static type load(const f16* p) { return *reinterpret_cast<const half4v*>(p); }
  __device__ static type zero() { return half4v{}; }
  __device__ static void store(f16* p, const float (&v)[4]) {
    *reinterpret_cast<half4v*>(p) = half4v{(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
  }
  __device__ static void store_raw(f16* p, type v) { *reinterpret_cast<half4v*>(p) = v; }
};
template <> struct Quad<float> {
  using type = float4v;
  __device__ static type load(const float* p) { return *reinterpret_cast<const float4v*>(p); }
  __device__ static type zero() { return float4v{0.f, 0.f, 0.f, 0.f}; }
  __device__ static void store(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4v*>(p) = float4v{v[0], v[1], v[2], v[3]};
  }
  __device__ static void store_raw(float* p, type v) { *reinterpret_cast<float4v*>(p) = v; }
};

template <typename T, int HP> struct DecTile;

// ------------------------------- f16 ----------------------------------------
// Lane l works on head hh = l % 16 and quarter g4 = l / 16.  Quad qi of the
// lane covers dims quad_dim(qi, g4) .. + 3 of the query, and of the output.
template <int HP> struct DecTile<f16, HP> {
  static constexpr int NS = HP / 32;  // 32-dim k-steps of the score MFMA
  static constexpr int NQ = HP / 16;  // quads per lane
  static constexpr int R = Ring<f16, HP>::value;
  half8v qf[NS];
  float4v o[NQ];
  half8v kf[R][NS];
  half8v vf[R][NS];

  __device__ static int quad_dim(int qi, int g4) { return 32 * (qi >> 1) + 8 * g4 + 4 * (qi & 1); }
  __device__ void init() {
#pragma unroll
    for (int e = 0; e < NQ; ++e) o[e] = float4v{0.f, 0.f, 0.f, 0.f};
  }
  // B operand of the score MFMA: lane l holds Q[hh][32s + 8 g4 + i], i < 8
  __device__ void set_q(const float (&x)[NQ][4]) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qf[s] = half8v{(f16)x[2 * s][0],     (f16)x[2 * s][1],     (f16)x[2 * s][2],
                     (f16)x[2 * s][3],     (f16)x[2 * s + 1][0], (f16)x[2 * s + 1][1],
                     (f16)x[2 * s + 1][2], (f16)x[2 * s + 1][3]};
  }
  // K and V rows j0 + l%16 (clamped to the last row of the run), dims
  // 32s + 8 g4 .. + 7; dims at or beyond H read as zero.
  template <int BUF>
  __device__ void load_kv(const f16* kb, const f16* vb, int j0, int last, int H, int lane) {
    const int g4 = lane >> 4;
    const int row = min(j0 + (lane & 15), last);
    const f16* kr = kb + (int64_t)row * H;
    const f16* vr = vb + (int64_t)row * H;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int d = 32 * s + 8 * g4;
      const int dc = d < H ? d : 0;
      half8v k = load_half8(kr + dc), v = load_half8(vr + dc);
      if (d >= H) {
        k = half8v{};
        v = half8v{};
      }
      kf[BUF][s] = k;
      vf[BUF][s] = v;
    }
  }
  // S^T[key j0 + 4 g4 + i][head hh] for i < 4
  template <int BUF>
  __device__ float4v scores() const {
    float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) acc = mfma16x16x32(kf[BUF][s], qf[s], acc);
    return acc;
  }
  __device__ void scale_o(float a) {
#pragma unroll
    for (int e = 0; e < NQ; ++e) o[e] *= a;
  }
  template <int BUF>
  __device__ void pv(const float4v& p, half4v ident) {
    const float4v zero = {0.f, 0.f, 0.f, 0.f};
    const half4v pb = {(f16)p[0], (f16)p[1], (f16)p[2], (f16)p[3]};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const half8v v = vf[BUF][s];
      const float4v tl = mfma16x16x16(half4v{v[0], v[1], v[2], v[3]}, ident, zero);
      const float4v th = mfma16x16x16(half4v{v[4], v[5], v[6], v[7]}, ident, zero);
      const half4v al = {(f16)tl[0], (f16)tl[1], (f16)tl[2], (f16)tl[3]};
      const half4v ah = {(f16)th[0], (f16)th[1], (f16)th[2], (f16)th[3]};
      o[2 * s] = mfma16x16x16(al, pb, o[2 * s]);
      o[2 * s + 1] = mfma16x16x16(ah, pb, o[2 * s + 1]);
    }
  }
};

// ------------------------------- f32 ----------------------------------------
template <int HP> struct DecTile<float, HP> {
  static constexpr int NQ = HP / 16;
  static constexpr int R = Ring<float, HP>::value;
  float qf[NQ][4];
  float4v o[NQ];
  float4v kf[R][NQ];
  float vf[R][4][NQ];

  __device__ static int quad_dim(int qi, int g4) { return 16 * qi + 4 * g4; }
  __device__ void init() {
#pragma unroll
    for (int t = 0; t < NQ; ++t) o[t] = float4v{0.f, 0.f, 0.f, 0.f};
  }
  // lane l: Q[hh][16t + 4 g4 + e]
  __device__ void set_q(const float (&x)[NQ][4]) {
#pragma unroll
    for (int t = 0; t < NQ; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[t][e] = x[t][e];
  }
  template <int BUF>
  __device__ void load_kv(const float* kb, const float* vb, int j0, int last, int H, int lane) {
    const int g4 = lane >> 4, l16 = lane & 15;
    const int krow = min(j0 + l16, last);
    const float* kr = kb + (int64_t)krow * H;
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      const int d = 16 * t + 4 * g4;
      float4v k = *reinterpret_cast<const float4v*>(kr + (d < H ? d : 0));
      kf[BUF][t] = (d < H) ? k : float4v{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int vrow = min(j0 + 4 * g4 + k, last);
      const float* vr = vb + (int64_t)vrow * H;
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        const int d = 16 * t + l16;
        const float v = vr[d < H ? d : 0];
        vf[BUF][k][t] = (d < H) ? v : 0.f;
      }
    }
  }
  template <int BUF>
  __device__ float4v scores() const {
    float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NQ; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mfma16x16x4f32(kf[BUF][t][e], qf[t][e], acc);
    return acc;
  }
  __device__ void scale_o(float a) {
#pragma unroll
    for (int t = 0; t < NQ; ++t) o[t] *= a;
  }
  template <int BUF>
  __device__ void pv(const float4v& p, half4v) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int t = 0; t < NQ; ++t) o[t] = mfma16x16x4f32(vf[BUF][k][t], p[k], o[t]);
  }
};

// ---------------------------------------------------------------------------
// lengths and the deal of waves
// ---------------------------------------------------------------------------
// Key count n of sample b, the row of its appended token (-1: none) and the
// first visible key (local window).
__device__ __forceinline__ void sample_keys(const DecodeParams& p, int b, int& n, int& newrow,
                                            int& kstart) {
  if (p.len_mode == 0) n = p.lens[b] + 1;
  else if (p.len_mode == 1) n = p.lens[0] + 1;
  else n = p.host_n;
  newrow = (p.k_new != nullptr) ? n - 1 : -1;
  if (n > p.cap) { n = p.cap; newrow = -1; }  // precondition violated: stay in bounds
  if (n < 0) { n = 0; newrow = -1; }
  kstart = (p.window >= 0) ? max(0, n - 1 - p.window) : 0;
}

__device__ __forceinline__ int sample_count(const DecodeParams& p, int b) {
  int n, newrow, kstart;
  sample_keys(p, b, n, newrow, kstart);
  return max(n - kstart, 0);
}

// Keys per wave: every unit gets ceil(c / quota) waves (at least one), with
// quota = max(64, ceil(K / (W - U))) for K live keys over U units and W waves,
// so the units never need more than W waves.  Called by all lanes of a wave.
__device__ int64_t deal_quota(const DecodeParams& p, int ups, int lane) {
  int64_t k = 0;
  for (int b = lane; b < p.B; b += 64) k += sample_count(p, b);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) k += __shfl_xor(k, m, 64);
  k *= ups;
  const int64_t units = (int64_t)p.B * ups;
  const int64_t spare = (int64_t)p.waves - units;
  if (spare <= 0) return INT64_MAX;
  return max(kMinKeysPerWave, (k + spare - 1) / spare);
}

__device__ __forceinline__ int waves_for(int c, int64_t quota) {
  if (c <= 0 || quota >= c) return 1;
  return (int)(((int64_t)c + quota - 1) / quota);
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_scan(int v, int lane) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int t = __shfl_up(v, m, 64);
    if (lane >= m) v += t;
  }
  return v;
}

// Sample served by global wave gw and the first wave of that sample's units;
// false when gw is beyond the waves in use.
__device__ bool find_sample(const DecodeParams& p, int ups, int64_t quota, int gw, int lane,
                            int& b_out, int& first_out) {
  int base = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int b = b0 + lane;
    const int v = (b < p.B) ? waves_for(sample_count(p, b), quota) * ups : 0;
    const int incl = wave_scan(v, lane);
    const bool hit = b < p.B && gw >= base + incl - v && gw < base + incl;
    const unsigned long long mask = __ballot(hit);
    if (mask != 0ull) {
      const int src = __ffsll((long long)mask) - 1;
      b_out = __shfl(b, src, 64);
      first_out = base + __shfl(incl - v, src, 64);
      return true;
    }
    base += __shfl(incl, 63, 64);
  }
  return false;
}

// First wave of sample b (all lanes of a wave call it).
__device__ int sample_first_wave(const DecodeParams& p, int ups, int64_t quota, int b, int lane) {
  int acc = 0;
  for (int b0 = 0; b0 < b; b0 += 64) {
    const int s = b0 + lane;
    acc += (s < b) ? waves_for(sample_count(p, s), quota) * ups : 0;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) acc += __shfl_xor(acc, m, 64);
  return acc;
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

// 1 / denominator of a merged (max m, sum l) pair with the optional sink
// logit sg, all in the log2 domain; 0 when no key was visible.
__device__ __forceinline__ float final_scale(float m, float l, bool has_sink, float sg) {
  if (l == 0.f) return 0.f;
  if (!has_sink) return 1.f / l;
  const float m2 = fmaxf(m, sg);
  const float den = l * fast_exp2(m - m2) + fast_exp2(sg - m2);
  return fast_exp2(m - m2) / den;
}

// Calls f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>) in order
// while f returns true.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_while(F&& f, std::integer_sequence<int, Is...>) {
  bool go = true;
  ((go = go && f(std::integral_constant<int, Is>{})), ...);
}

// FEAT bits: kSoftcap (scores are soft-capped), kExtras (additive bias and/or
// mask, and/or the qk output).  The plain variant has no per-score checks.
constexpr int kSoftcap = 1, kExtras = 2;

template <typename T, int HP, int FEAT>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(DecodeParams p) {
  using Tile = DecTile<T, HP>;
  using Q4 = Quad<T>;
  using QT = typename Q4::type;
  constexpr int NQ = HP / 16, NH = NQ / 2, R = Tile::R;

  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6);
  const int H = p.H;
  const int g = p.N / p.kvN;
  const int hg = p.head_groups;
  const int ups = p.kvN * hg;

  // ---- which unit and which run of its keys ---------------------------------
  const int64_t quota = deal_quota(p, ups, lane);
  int b, first;
  if (!find_sample(p, ups, quota, gw, lane, b, first)) return;  // idle wave
  int n, newrow, kstart;
  sample_keys(p, b, n, newrow, kstart);
  const int c = max(n - kstart, 0);
  const int wb = waves_for(c, quota);
  const int local = gw - first;
  const int ui = local / wb, part = local % wb;
  const int kvh = ui / hg, hgrp = ui % hg;
  const int h0 = kvh * g + hgrp * 16;
  const int nh = min(16, g - hgrp * 16);
  const int j_begin = kstart + (int)((int64_t)c * part / wb);
  const int j_end = kstart + (int)((int64_t)c * (part + 1) / wb);
  const int nsub = (j_end - j_begin + 15) / 16;
  const int last = j_end - 1;
  const bool append = newrow >= j_begin && newrow < j_end;

  T* kb = static_cast<T*>(p.kc) + ((int64_t)b * p.kvN + kvh) * p.cap * H;
  T* vb = static_cast<T*>(p.vc) + ((int64_t)b * p.kvN + kvh) * p.cap * H;
  const int half = H / 2;
  const T* cs = static_cast<const T*>(p.cos);
  const T* sn = static_cast<const T*>(p.sin);
  const bool rot = cs != nullptr;
  const int pos = min(max(n - 1, 0), max(p.rot_rows - 1, 0));  // rotary row of the new token
  const T* cs_row = rot ? cs + (int64_t)pos * half : nullptr;
  const T* sn_row = rot ? sn + (int64_t)pos * half : nullptr;

  // ---- the query: RMSNorm and rotary in registers ------------------------------
  // x[qi][e] = query element quad_dim(qi, g4) + e of head h0 + hh.  With H
  // equal to the padded size both members of a rotary pair (d, d + H/2) are
  // quads qi and qi + NQ/2 of the same lane and the set-up is split: its
  // loads go out before the first key/value loads, its arithmetic runs while
  // those are in flight.  Other head sizes load the partner quads and finish
  // the set-up before streaming starts.
  const int hh = lane & 15, g4 = lane >> 4;
  const T* qrow = static_cast<const T*>(p.q) + ((int64_t)b * p.N + h0 + min(hh, nh - 1)) * H;
  const T* qw = static_cast<const T*>(p.q_norm);
  const bool same_lane_pairs = (H == HP);
  float x[NQ][4];
  auto load_quads = [&](QT (&dst)[NQ], const T* src, bool on) {
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      const int d = Tile::quad_dim(qi, g4);
      dst[qi] = (on && d < H) ? Q4::load(src + d) : Q4::zero();
    }
  };
  // RMSNorm of x (sum over the four lanes of a head); returns the factor
  auto norm_x = [&](const QT (&w)[NQ]) -> float {
    float ss = 0.f;
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += x[qi][e] * x[qi][e];
    ss += shfl_xor(ss, 16);
    ss += shfl_xor(ss, 32);
    const float r = rsqrtf(ss / (float)H + p.eps);
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[qi][e] *= r * to_f32(w[qi][e]);
    return r;
  };
  QT qr[NQ], wr[NQ], cr[NH], sr[NH];
  if (same_lane_pairs) {
    load_quads(qr, qrow, true);
    load_quads(wr, qw, qw != nullptr);
    if (rot) {
#pragma unroll
      for (int qi = 0; qi < NH; ++qi) {
        const int d = Tile::quad_dim(qi, g4);  // < H / 2
        cr[qi] = Q4::load(cs_row + d);
        sr[qi] = Q4::load(sn_row + d);
      }
    }
  } else {
    QT raw[NQ];
    load_quads(raw, qrow, true);
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[qi][e] = to_f32(raw[qi][e]);
    float rn = 1.f;
    if (qw != nullptr) {
      load_quads(raw, qw, true);
      rn = norm_x(raw);
    }
    if (rot) {
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) {
        const int d = Tile::quad_dim(qi, g4);
        if (d < H) {
          const int i = d < half ? d : d - half;
          const int dp = d < half ? d + half : d - half;
          const QT zq = Q4::load(qrow + dp);
          const QT zw = qw != nullptr ? Q4::load(qw + dp) : Q4::zero();
          const QT co = Q4::load(cs_row + i), si = Q4::load(sn_row + i);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float z = to_f32(zq[e]);
            if (qw != nullptr) z *= rn * to_f32(zw[e]);
            const float c0 = to_f32(co[e]), s0 = to_f32(si[e]);
            x[qi][e] = d < half ? x[qi][e] * c0 - z * s0 : x[qi][e] * c0 + z * s0;
          }
        }
      }
    }
  }

  // the appended row: lane l holds dims 4l .. 4l + 3 (H <= 256)
  const int ad = 4 * lane;
  const bool alane = ad < H;
  QT ak = Q4::zero(), av = Q4::zero(), aw = Q4::zero(), ac = Q4::zero(), as = Q4::zero();
  if (append && alane) {
    const int64_t nrow = ((int64_t)b * p.kvN + kvh) * H;
    ak = Q4::load(static_cast<const T*>(p.k_new) + nrow + ad);
    av = Q4::load(static_cast<const T*>(p.v_new) + nrow + ad);
    if (p.k_norm != nullptr) aw = Q4::load(static_cast<const T*>(p.k_norm) + ad);
    if (rot) {
      const int i = ad < half ? ad : ad - half;
      ac = Q4::load(cs_row + i);
      as = Q4::load(sn_row + i);
    }
  }
  auto do_append = [&]() {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = to_f32(ak[e]);
    if (p.k_norm != nullptr) {
      float ss = y[0] * y[0] + y[1] * y[1] + y[2] * y[2] + y[3] * y[3];
      ss = wave_sum_xor(ss, 1, 32);
      const float r = rsqrtf(ss / (float)H + p.eps);
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] *= r * to_f32(aw[e]);
    }
    if (rot) {
      const int src = alane ? (ad < half ? lane + H / 8 : lane - H / 8) : lane;
      float yp[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) yp[e] = __shfl(y[e], src, 64);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float co = to_f32(ac[e]), si = to_f32(as[e]);
        y[e] = ad < half ? y[e] * co - yp[e] * si : y[e] * co + yp[e] * si;
      }
    }
    if (alane) {
      Q4::store(kb + (int64_t)newrow * H + ad, y);
      Q4::store_raw(vb + (int64_t)newrow * H + ad, av);
    }
    // the row is read back by other lanes of this wave: order the stores
    // before those loads (no instruction is needed within one wave)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // ---- start streaming --------------------------------------------------------
  auto jof = [&](int k) { return j_begin + 16 * k; };
  const bool append_early = append && (newrow - j_begin) / 16 < R - 1;
  if (append_early) do_append();
  Tile tile;
  tile.init();
  static_for_while(
      [&](auto rt) -> bool {
        constexpr int r = decltype(rt)::value;
        if (r >= nsub) return false;
        tile.template load_kv<r>(kb, vb, jof(r), last, H, lane);
        return true;
      },
      std::make_integer_sequence<int, R - 1>{});
  if (append && !append_early) do_append();

  if (same_lane_pairs) {
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[qi][e] = to_f32(qr[qi][e]);
    if (qw != nullptr) norm_x(wr);
    if (rot) {
#pragma unroll
      for (int qi = 0; qi < NH; ++qi)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float co = to_f32(cr[qi][e]), si = to_f32(sr[qi][e]);
          const float a = x[qi][e], z = x[qi + NH][e];
          x[qi][e] = a * co - z * si;
          x[qi + NH][e] = z * co + a * si;
        }
    }
  }
  tile.set_q(x);

  // identity for the f16 V transpose: lane l holds B[k = 4(l/16)+i][n = l%16]
  half4v ident;
#pragma unroll
  for (int i = 0; i < 4; ++i) ident[i] = (f16)((4 * g4 + i) == hh ? 1.f : 0.f);

  const bool head_ok = hh < nh;
  const int h = h0 + hh;
  const float scale = p.scale;
  const float cap = p.softcap, inv_cap = p.softcap > 0.f ? 1.f / p.softcap : 0.f;
  const T* bias = static_cast<const T*>(p.bias);
  T* qk = static_cast<T*>(p.qk);

  float m = kNegInf, l = 0.f;
  // Score transform, online softmax and PV for the sub-tile held in BUF.
  auto process = [&](auto buf_tag, int j0) {
    constexpr int BUF = decltype(buf_tag)::value;
    const float4v sc = tile.template scores<BUF>();
    mfma_result_fence();
    float tmax = kNegInf;
    float4v x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = j0 + 4 * g4 + i;
      const bool ok = head_ok && key < j_end;
      float v = sc[i] * scale;
      if (FEAT & kSoftcap) v = softcap_apply(v, cap, inv_cap);
      if (FEAT & kExtras) {
        if (ok && bias != nullptr && key < p.bias_cols)
          v += to_f32(bias[b * p.bias_sb + h * p.bias_sh + key]);
        if (ok && p.mask != nullptr && key < p.mask_cols)
          v += (p.mask[(int64_t)b * p.mask_cols + key] == 0) ? p.mask_filter : 0.f;
        if (ok && qk != nullptr) qk[((int64_t)b * p.N + h) * p.host_n + key] = from_f32<T>(v);
      }
      v = ok ? v * kLog2e : kNegInf;
      x[i] = v;
      tmax = fmaxf(tmax, v);
    }
    tmax = fmaxf(tmax, shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const float mnew = fmaxf(m, tmax);
    const float muse = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = fast_exp2(m - muse);
    m = mnew;
    float4v pr;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = fast_exp2(x[i] - muse);
      pr[i] = e;
      psum += e;
    }
    l = l * alpha + psum;
    tile.scale_o(alpha);
    tile.template pv<BUF>(pr, ident);
  };

  // The ring: sub-tile k lives in buffer k % R; the load of sub-tile k + R - 1
  // is issued before sub-tile k is computed.
  for (int k = 0; k < nsub; k += R) {
    static_for_while(
        [&](auto rt) -> bool {
          constexpr int r = decltype(rt)::value;
          const int kk = k + r;
          if (kk >= nsub) return false;
          if (kk + R - 1 < nsub)
            tile.template load_kv<(r + R - 1) % R>(kb, vb, jof(kk + R - 1), last, H, lane);
          process(std::integral_constant<int, r>{}, jof(kk));
          return true;
        },
        std::make_integer_sequence<int, R>{});
  }
  mfma_result_fence();
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  if (!head_ok) return;

  // ---- output (single wave per unit) or partial ---------------------------------
  if (wb == 1) {
    bool has;
    const float sg = read_sink<T>(p, h, has);
    const float inv = final_scale(m, l, has, sg);
    T* orow = static_cast<T*>(p.out) + ((int64_t)b * p.N + h) * H;
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      const int d = Tile::quad_dim(qi, g4);
      if (d < H) {
        const float v[4] = {tile.o[qi][0] * inv, tile.o[qi][1] * inv, tile.o[qi][2] * inv,
                            tile.o[qi][3] * inv};
        Q4::store(orow + d, v);
      }
    }
  } else {
    float* rec = p.part + ((int64_t)gw * p.hpw + hh) * (HP + 4);
    if (g4 == 0) *reinterpret_cast<float2v*>(rec) = float2v{m, l};
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      const int d = Tile::quad_dim(qi, g4);
      if (d < H) *reinterpret_cast<float4v*>(rec + 4 + d) = tile.o[qi];
    }
  }
}

// Merge the partials of one (sample, query head): a first pass over the
// partials' (max, sum) pairs, then every thread sums one quad of dims over a
// stride of the partials, and the strides are added in LDS.
template <typename T, int HP>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
  constexpr int NQD = HP / 4;            // quads of a padded head
  constexpr int NG = 256 / NQD;          // partial strides
  __shared__ float red_m[4], red_l[4];
  __shared__ float4v acc_s[NG][NQD];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = p.N / p.kvN, hg = p.head_groups, ups = p.kvN * hg;
  const int64_t quota = deal_quota(p, ups, lane);
  const int wb = waves_for(sample_count(p, b), quota);
  if (wb <= 1) return;  // written directly
  const int first = sample_first_wave(p, ups, quota, b, lane);
  const int kvh = h / g, hgrp = (h % g) / 16, hh = (h % g) % 16;
  const int w0 = first + (kvh * hg + hgrp) * wb;
  auto rec = [&](int i) { return p.part + ((int64_t)(w0 + i) * p.hpw + hh) * (HP + 4); };

  // pass 1: M = max m_i, L = sum l_i 2^(m_i - M)
  float M = kNegInf, L = 0.f;
  for (int i = tid; i < wb; i += 256) {
    const float2v ml = *reinterpret_cast<const float2v*>(rec(i));
    const float mn = fmaxf(M, ml[0]);
    const float mu = (mn == kNegInf) ? 0.f : mn;
    L = L * fast_exp2(M - mu) + ml[1] * fast_exp2(ml[0] - mu);
    M = mn;
  }
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const float m2 = shfl_xor(M, s), l2 = shfl_xor(L, s);
    const float mn = fmaxf(M, m2);
    const float mu = (mn == kNegInf) ? 0.f : mn;
    L = L * fast_exp2(M - mu) + l2 * fast_exp2(m2 - mu);
    M = mn;
  }
  if (lane == 0) {
    red_m[wave] = M;
    red_l[wave] = L;
  }
  __syncthreads();
  M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  const float Mu = (M == kNegInf) ? 0.f : M;
  L = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) L += red_l[w] * fast_exp2(red_m[w] - Mu);

  // pass 2: sum of o_i 2^(m_i - M) per quad of dims
  const int dq = tid % NQD, gs = tid / NQD;
  float4v acc = {0.f, 0.f, 0.f, 0.f};
  if (4 * dq < p.H) {
#pragma unroll 4
    for (int i = gs; i < wb; i += NG) {
      const float* r = rec(i);
      const float f = fast_exp2(r[0] - Mu);
      acc += *reinterpret_cast<const float4v*>(r + 4 + 4 * dq) * f;
    }
  }
  acc_s[gs][dq] = acc;
  __syncthreads();
  if (tid < NQD && 4 * tid < p.H) {
    float4v o = acc_s[0][tid];
#pragma unroll
    for (int s = 1; s < NG; ++s) o += acc_s[s][tid];
    bool has;
    const float sg = read_sink<T>(p, h, has);
    const float inv = final_scale(M, L, has, sg);
    const float v[4] = {o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    Quad<T>::store(static_cast<T*>(p.out) + ((int64_t)b * p.N + h) * p.H + 4 * tid, v);
  }
}

template <typename T, int HP, int FEAT>
hipError_t launch_decode_f(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<T, HP, FEAT>), dim3(p.waves / kWavesPerGroup), dim3(kThreads),
                     0, s, p);
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

template <typename T, int HP>
hipError_t launch_combine_t(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL((decode_combine_kernel<T, HP>), dim3(p.N, p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(DType dt, int hp, const DecodeParams& p, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  if (dt == DType::F16) {
    if (hp == 64) return launch_decode_t<f16, 64>(p, s);
    if (hp == 128) return launch_decode_t<f16, 128>(p, s);
    return launch_decode_t<f16, 256>(p, s);
  }
  if (hp == 64) return launch_decode_t<float, 64>(p, s);
  if (hp == 128) return launch_decode_t<float, 128>(p, s);
  return launch_decode_t<float, 256>(p, s);
}

// Needed only when some unit may be served by more than one wave, i.e. when
// the grid has more waves than units.
hipError_t launch_decode_combine(DType dt, int hp, const DecodeParams& p, hipStream_t s) {
  if (p.B == 0 || (int64_t)p.waves <= (int64_t)p.B * p.kvN * p.head_groups) return hipSuccess;
  if (dt == DType::F16) {
    if (hp == 64) return launch_combine_t<f16, 64>(p, s);
    if (hp == 128) return launch_combine_t<f16, 128>(p, s);
    return launch_combine_t<f16, 256>(p, s);
  }
  if (hp == 64) return launch_combine_t<float, 64>(p, s);
  if (hp == 128) return launch_combine_t<float, 128>(p, s);
  return launch_combine_t<float, 256>(p, s);
}

}  // namespace kvattn
