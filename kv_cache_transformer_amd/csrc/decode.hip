// K3: single-token attention over a BNSH cache (GroupQueryAttention decode,
// DecoderMaskedMultiHeadAttention self and cross attention).
//
// Work split (GroupQueryAttention page, Implementation variants: decode is
// partitioned along the key axis and the partial online-softmax results are
// merged).  A unit is (sample b, kv head, group of <= 16 query heads sharing
// that kv head).  The live keys of all units are dealt out to pairs of waves
// so that every pair streams about the same number of key rows, each unit
// receiving a whole number of pairs (at least one) and each pair a contiguous
// run of its keys.  The lengths are device data, so every wave derives the
// deal from them itself.
//
// A workgroup is eight waves on one CU; waves j and j + 4 share a SIMD and
// form pair j.  Of two waves on a SIMD the older one wins the memory-issue
// arbitration and the younger one gets what is left (measured: about 60 % of
// the rate, and the issue priority does not change it), so the two waves of
// a pair do not split their run statically: the run is cut into chunks that
// they claim from an LDS counter.  Each chunk's partial (max, sum,
// unnormalised output per head) goes to its own LDS record and the pair
// merges them in chunk order, so the result does not depend on which wave
// took which chunk.  A unit served by one pair gets its output from that
// pair.  Otherwise each pair writes one partial per head to the workspace and
// counts its arrival on the unit's counter; the pair that arrives last merges
// the unit's partials in pair order with a log-sum-exp combine, adds the
// head-sink term, writes the output and sets the counter back to zero (the
// merge dispatch the page describes is folded into this one launch).  A wave
// reads its rows of the cache once for all query heads of its unit, with up
// to three 16-row sub-tiles in flight in a register ring.
//
// The query (optionally RMS-normed per head, then NeoX-rotated at the new
// token's position) is built in registers in the MFMA operand layout before
// the wave issues its first key/value load.  The new token's key (normed and
// rotated the same way) and value are appended by the wave whose run holds
// the new row, before that wave loads the row (GroupQueryAttention page,
// Inputs table: past_key/present_key, q/k_norm_weight, cos/sin_cache).  Lanes
// of one wave see each other's global stores in program order, so no barrier
// is needed.
//
// MFMA mapping per 16-key sub-tile (wave64):
//   S^T[16 keys][16 heads] = K[16][H] . Q^T      (f16: 16x16x32, f32: 16x16x4)
//   O^T[H][16 heads]      += V^T[H][16] . P^T    (f16: 16x16x16, f32: 16x16x4)
// For f16 the V^T fragments come from an identity MFMA on the row-major V
// fragment (exact: products with 1 and sums with 0), so V needs no LDS.
//
// int8 caches (GroupQueryAttention page, Attributes table: k/v_quant_type,
// kv_cache_bit_width 8; Inputs table: k_scale, v_scale; float32 activations)
// run the f16 tile on the codes, which f16 holds exactly: the key scales are
// folded into the query, a power of two per head brings its largest element
// into [2^13, 2^14), and the query and the probabilities (times 2^12) are
// each split into two f16 terms hi + lo, so that the products stay within
// float32 rounding of the float32 computation.  The value scales and 2^-12
// are applied once per pair, to its merged output.  The appended row is
// quantised in place: code = clamp(rint(x / scale)) with the float32 quotient.
#include <type_traits>
#include <utility>

#include "device_common.hpp"
#include "kvattn_internal.hpp"

namespace kvattn {
namespace {

constexpr int kThreads = 512;
constexpr int kWavesPerGroup = kThreads / 64;
constexpr int kPairsPerGroup = kWavesPerGroup / 2;
// LDS for the chunk partials of a workgroup's pairs (floats), and the most
// chunks a pair's run is cut into
constexpr int kPartFloats = 30720;
constexpr int kMaxChunks = 16;
constexpr int64_t kMinKeysPerWave = 64;
// s_waitcnt immediate for vmcnt(0) with the other counters unconstrained
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;

// Slack of the running maximum (log2 units): probabilities stay <= 2^3, which
// the int8 tile's 2^12-scaled f16 split holds (2^15 < 65504).
constexpr float kDecodeSlack = 3.f;

// Cache type tags: float32 activations (query, new rows, output) over an int8
// key/value cache, or over an int4 one (two codes per byte).
struct QuantI8 {};
struct QuantI4 {};
template <typename T> struct ActOf { using type = T; };
template <> struct ActOf<QuantI8> { using type = float; };
template <> struct ActOf<QuantI4> { using type = float; };
template <typename T> struct CacheOf { using type = T; };
template <> struct CacheOf<QuantI8> { using type = int8_t; };
template <> struct CacheOf<QuantI4> { using type = uint8_t; };

// Register ring depth (16-row sub-tiles held per wave): R - 1 are in flight
// while one is computed, sized to stay within 256 registers without spilling.
template <typename T, int HP> struct Ring { static constexpr int value = 1; };
template <> struct Ring<f16, 64> { static constexpr int value = 4; };
template <> struct Ring<f16, 128> { static constexpr int value = 4; };
template <> struct Ring<float, 64> { static constexpr int value = 3; };
template <> struct Ring<QuantI8, 64> { static constexpr int value = 4; };
template <> struct Ring<QuantI8, 128> { static constexpr int value = 4; };
template <> struct Ring<QuantI8, 256> { static constexpr int value = 1; };
template <> struct Ring<QuantI4, 64> { static constexpr int value = 4; };
template <> struct Ring<QuantI4, 128> { static constexpr int value = 4; };
template <> struct Ring<QuantI4, 256> { static constexpr int value = 1; };

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

// Compiler barrier on a register value: what uses v after this point cannot
// be moved above it (used to keep conversions of loaded values inside the
// branch that needs them, so other paths never wait for those loads).
template <typename V>
__device__ __forceinline__ void pin(V& v) {
  asm volatile("" : "+v"(v));
}

template <typename T, int HP, int R> struct DecTile;

// ------------------------------- f16 ----------------------------------------
// Lane l works on head hh = l % 16 and quarter g4 = l / 16.  Quad qi of the
// lane covers dims quad_dim(qi, g4) .. + 3 of the query, and of the output.
template <int HP, int R> struct DecTile<f16, HP, R> {
  static constexpr int NS = HP / 32;  // 32-dim k-steps of the score MFMA
  static constexpr int NQ = HP / 16;  // quads per lane
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
  // 32s + 8 g4 .. + 7.  Slots at or beyond H re-read dims 0..7 of the row:
  // the query is zero there, so they add nothing to the scores, and those
  // output dims are never stored.  (Masking the loaded values would make
  // every load wait for its data at once.)
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
      kf[BUF][s] = load_half8(kr + dc);
      vf[BUF][s] = load_half8(vr + dc);
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
template <int HP, int R> struct DecTile<float, HP, R> {
  static constexpr int NQ = HP / 16;
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
    // slots at or beyond H re-read the row's first dims (see the f16 tile)
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
      const int d = 16 * t + 4 * g4;
      kf[BUF][t] = *reinterpret_cast<const float4v*>(kr + (d < H ? d : 0));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int vrow = min(j0 + 4 * g4 + k, last);
      const float* vr = vb + (int64_t)vrow * H;
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        const int d = 16 * t + l16;
        vf[BUF][k][t] = vr[d < H ? d : 0];
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

// ------------------------------ int8 ----------------------------------------
// Eight int8 codes as f16.  Each byte u = code + 128 (sign bit flipped)
// becomes the low mantissa byte of 1024.0 (0x6400 | u = 1024 + u, exact),
// and 1152 is subtracted (exact).
__device__ __forceinline__ half8v codes_to_half8(uint2v w) {
  half8v out;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t a = w[k] ^ 0x80808080u;
    // v_perm_b32: selector bytes 0-3 take bytes of the second operand, 4-7 of
    // the first: (a.b0, 0x64, a.b1, 0x64) and (a.b2, 0x64, a.b3, 0x64)
    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, a, 0x04010400u);
    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, a, 0x04030402u);
    const half2v l2 = __builtin_bit_cast(half2v, lo) - half2v{(f16)1152.f, (f16)1152.f};
    const half2v h2 = __builtin_bit_cast(half2v, hi) - half2v{(f16)1152.f, (f16)1152.f};
    out[4 * k] = l2[0];
    out[4 * k + 1] = l2[1];
    out[4 * k + 2] = h2[0];
    out[4 * k + 3] = h2[1];
  }
  return out;
}

// Code of x for scale s at 8 bits: the float32 quotient rounded half to even,
// clamped to [-128, 127].
__device__ __forceinline__ uint32_t quant8(float x, float s) {
  const float c = fminf(fmaxf(rintf(x / s), -128.f), 127.f);
  return (uint32_t)(int)c & 0xFFu;
}

// ------------------------------ int4 ----------------------------------------
// Eight int4 codes of one 32-bit word (byte i: dim 2i in the low nibble, dim
// 2i + 1 in the high one, each stored as code + 8) as f16: the nibbles are
// spread to one byte each in dim order, each byte becomes the low mantissa
// bits of 1024.0 (0x6400 | u = 1024 + u, exact) and 1032 is subtracted
// (exact).  v_perm_b32: selector bytes 0-3 take bytes of the second operand,
// 4-7 of the first.
__device__ __forceinline__ half8v nibbles_to_half8(uint32_t w) {
  const uint32_t ev = w & 0x0F0F0F0Fu;                              // byte k: dim 2k
  const uint32_t od = (w >> 4) & 0x0F0F0F0Fu;                       // byte k: dim 2k + 1
  const uint32_t d03 = __builtin_amdgcn_perm(od, ev, 0x05010400u);  // dims 0, 1, 2, 3
  const uint32_t d47 = __builtin_amdgcn_perm(od, ev, 0x07030602u);  // dims 4, 5, 6, 7
  half8v out;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t a = k ? d47 : d03;
    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, a, 0x04010400u);
    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, a, 0x04030402u);
    const half2v l2 = __builtin_bit_cast(half2v, lo) - half2v{(f16)1032.f, (f16)1032.f};
    const half2v h2 = __builtin_bit_cast(half2v, hi) - half2v{(f16)1032.f, (f16)1032.f};
    out[4 * k] = l2[0];
    out[4 * k + 1] = l2[1];
    out[4 * k + 2] = h2[0];
    out[4 * k + 3] = h2[1];
  }
  return out;
}

// Stored nibble of x for scale s at 4 bits: the float32 quotient rounded half
// to even, clamped to [-8, 7], plus 8.
__device__ __forceinline__ uint32_t quant4(float x, float s) {
  const float c = fminf(fmaxf(rintf(x / s), -8.f), 7.f);
  return (uint32_t)((int)c + 8);
}

// Lane layout as the f16 tile (lane l: key row l % 16, quarter g4 = l / 16),
// the codes packed in the ring and widened when used.  For HP >= 128 a lane
// loads 16 codes at a time, dims 64 i + 16 g4 .. + 15 (two k-steps: load i
// serves k-steps 2i and 2i + 1), which keeps the rotary partners d, d + HP/2
// in quads qi, qi + NQ/2 of one lane.  A load that would cross the row's end
// (H not a multiple of 16) starts 8 codes early instead; that lane then
// labels its k-steps the other way round (the early half stands for dims past
// the head, where the query is zero and no output is stored).  HP = 64 keeps
// 8-code loads (dims 32 s + 8 g4 .. + 7).
template <int HP, int R> struct DecTile<QuantI8, HP, R> {
  static constexpr int NS = HP / 32;  // 32-dim k-steps of the score MFMA
  static constexpr int NQ = HP / 16;  // quads per lane
  static constexpr bool kWide = HP >= 128;
  static constexpr int NL = kWide ? HP / 64 : NS;  // loads per matrix and sub-tile
  using Raw = typename std::conditional<kWide, uint4v, uint2v>::type;
  static constexpr float kPScale = 4096.f;  // probabilities are split at 2^12 scale
  half8v qh[NS], ql[NS];
  float4v o[NQ];
  Raw kr[R][NL];
  Raw vr[R][NL];
  uint32_t swap = 0;  // bit i: load i starts 8 codes early (its k-steps are exchanged)

  __device__ int quad_dim(int qi, int g4) const {
    if constexpr (kWide) {
      const int i = qi >> 2;
      const int j = ((qi >> 1) & 1) ^ (int)((swap >> i) & 1u);
      return 64 * i + 16 * g4 + 8 * j + 4 * (qi & 1);
    } else {
      return 32 * (qi >> 1) + 8 * g4 + 4 * (qi & 1);
    }
  }
  __device__ void set_layout(int H, int lane) {
    swap = 0;
    if constexpr (kWide) {
      const int g4 = lane >> 4;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int d = 64 * i + 16 * g4;
        if (d < H && d + 16 > H) swap |= 1u << i;
      }
    }
  }
  __device__ void init() {
#pragma unroll
    for (int e = 0; e < NQ; ++e) o[e] = float4v{0.f, 0.f, 0.f, 0.f};
  }
  // x: the query with the key scales folded in, scaled by a power of two;
  // hi = f16(x), lo = f16(x - hi)
  __device__ void set_q(const float (&x)[NQ][4]) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = x[2 * s + (i >> 2)][i & 3];
        const f16 h = (f16)v;
        qh[s][i] = h;
        ql[s][i] = (f16)(v - (float)h);
      }
  }
  // Rows j0 + l % 16 (clamped to the last row of the run); every load stays
  // inside its row (slots past the head re-read the row's first codes).
  template <int BUF>
  __device__ void load_kv(const int8_t* kb, const int8_t* vb, int j0, int last, int H, int lane) {
    const int g4 = lane >> 4;
    const int row = min(j0 + (lane & 15), last);
    const int8_t* krow = kb + (int64_t)row * H;
    const int8_t* vrow = vb + (int64_t)row * H;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      int off;
      if constexpr (kWide) {
        const int d = 64 * i + 16 * g4;
        off = d + 16 <= H ? d : (d < H ? d - 8 : 0);
      } else {
        const int d = 32 * i + 8 * g4;
        off = d < H ? d : 0;
      }
      kr[BUF][i] = *reinterpret_cast<const Raw*>(krow + off);
      vr[BUF][i] = *reinterpret_cast<const Raw*>(vrow + off);
    }
  }
  // the 8 codes of k-step s
  __device__ static uint2v step_codes(const Raw (&r)[NL], int s) {
    if constexpr (kWide) {
      const uint4v w = r[s >> 1];
      return (s & 1) ? uint2v{w[2], w[3]} : uint2v{w[0], w[1]};
    } else {
      return r[s];
    }
  }
  template <int BUF>
  __device__ float4v scores() const {
    float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const half8v k = codes_to_half8(step_codes(kr[BUF], s));
      acc = mfma16x16x32(k, qh[s], acc);
      acc = mfma16x16x32(k, ql[s], acc);
    }
    return acc;
  }
  __device__ void scale_o(float a) {
#pragma unroll
    for (int e = 0; e < NQ; ++e) o[e] *= a;
  }
  template <int BUF>
  __device__ void pv(const float4v& p, half4v ident) {
    const float4v zero = {0.f, 0.f, 0.f, 0.f};
    half4v ph, pl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = p[i] * kPScale;
      ph[i] = (f16)v;
      pl[i] = (f16)(v - (float)ph[i]);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const half8v v = codes_to_half8(step_codes(vr[BUF], s));
      const float4v tl = mfma16x16x16(half4v{v[0], v[1], v[2], v[3]}, ident, zero);
      const float4v th = mfma16x16x16(half4v{v[4], v[5], v[6], v[7]}, ident, zero);
      const half4v al = {(f16)tl[0], (f16)tl[1], (f16)tl[2], (f16)tl[3]};
      const half4v ah = {(f16)th[0], (f16)th[1], (f16)th[2], (f16)th[3]};
      o[2 * s] = mfma16x16x16(al, ph, o[2 * s]);
      o[2 * s] = mfma16x16x16(al, pl, o[2 * s]);
      o[2 * s + 1] = mfma16x16x16(ah, ph, o[2 * s + 1]);
      o[2 * s + 1] = mfma16x16x16(ah, pl, o[2 * s + 1]);
    }
  }
};

// int4: the int8 tile's arithmetic on nibble codes.  A lane loads two runs of
// HP/8 codes per row, dims (HP/2) i + (HP/8) g4 .. + HP/8 - 1 for i = 0, 1
// (HP/16 bytes each), so that the rotary partners d and d + HP/2 are quads qi
// and qi + NQ/2 of one lane; 32-bit word w of run i holds the eight codes of
// k-step i (NS/2) + w.  A run lies inside the head or wholly past it (the head
// size is a multiple of HP/8); runs past it re-read the row's first bytes
// (the query is zero there and those outputs are not stored).
template <int HP, int R> struct DecTile<QuantI4, HP, R> {
  static constexpr int NS = HP / 32;  // 32-dim k-steps of the score MFMA
  static constexpr int NQ = HP / 16;  // quads per lane
  static constexpr int WPR = NS / 2;  // 32-bit words per run
  using Raw = typename std::conditional<WPR == 1, uint32_t,
                                        typename std::conditional<WPR == 2, uint2v, uint4v>::type>::type;
  static constexpr float kPScale = 4096.f;  // probabilities are split at 2^12 scale
  half8v qh[NS], ql[NS];
  float4v o[NQ];
  Raw kr[R][2];
  Raw vr[R][2];

  __device__ int quad_dim(int qi, int g4) const {
    const int s = qi >> 1;
    return (HP / 2) * (s / WPR) + (HP / 8) * g4 + 8 * (s % WPR) + 4 * (qi & 1);
  }
  __device__ void set_layout(int, int) {}
  __device__ void init() {
#pragma unroll
    for (int e = 0; e < NQ; ++e) o[e] = float4v{0.f, 0.f, 0.f, 0.f};
  }
  // as the int8 tile: hi = f16(x), lo = f16(x - hi)
  __device__ void set_q(const float (&x)[NQ][4]) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = x[2 * s + (i >> 2)][i & 3];
        const f16 h = (f16)v;
        qh[s][i] = h;
        ql[s][i] = (f16)(v - (float)h);
      }
  }
  // Rows j0 + l % 16 (clamped to the last row of the run), H / 2 bytes each.
  template <int BUF>
  __device__ void load_kv(const uint8_t* kb, const uint8_t* vb, int j0, int last, int H, int lane) {
    const int g4 = lane >> 4;
    const int row = min(j0 + (lane & 15), last);
    const uint8_t* krow = kb + (int64_t)row * (H / 2);
    const uint8_t* vrow = vb + (int64_t)row * (H / 2);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int d = (HP / 2) * i + (HP / 8) * g4;
      const int off = d < H ? d / 2 : 0;
      kr[BUF][i] = *reinterpret_cast<const Raw*>(krow + off);
      vr[BUF][i] = *reinterpret_cast<const Raw*>(vrow + off);
    }
  }
  // the 8 codes of k-step s
  __device__ static uint32_t step_word(const Raw (&r)[2], int s) {
    if constexpr (WPR == 1) {
      return r[s];
    } else {
      return r[s / WPR][s % WPR];
    }
  }
  template <int BUF>
  __device__ float4v scores() const {
    float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const half8v k = nibbles_to_half8(step_word(kr[BUF], s));
      acc = mfma16x16x32(k, qh[s], acc);
      acc = mfma16x16x32(k, ql[s], acc);
    }
    return acc;
  }
  __device__ void scale_o(float a) {
#pragma unroll
    for (int e = 0; e < NQ; ++e) o[e] *= a;
  }
  template <int BUF>
  __device__ void pv(const float4v& p, half4v ident) {
    const float4v zero = {0.f, 0.f, 0.f, 0.f};
    half4v ph, pl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = p[i] * kPScale;
      ph[i] = (f16)v;
      pl[i] = (f16)(v - (float)ph[i]);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const half8v v = nibbles_to_half8(step_word(vr[BUF], s));
      const float4v tl = mfma16x16x16(half4v{v[0], v[1], v[2], v[3]}, ident, zero);
      const float4v th = mfma16x16x16(half4v{v[4], v[5], v[6], v[7]}, ident, zero);
      const half4v al = {(f16)tl[0], (f16)tl[1], (f16)tl[2], (f16)tl[3]};
      const half4v ah = {(f16)th[0], (f16)th[1], (f16)th[2], (f16)th[3]};
      o[2 * s] = mfma16x16x16(al, ph, o[2 * s]);
      o[2 * s] = mfma16x16x16(al, pl, o[2 * s]);
      o[2 * s + 1] = mfma16x16x16(ah, ph, o[2 * s + 1]);
      o[2 * s + 1] = mfma16x16x16(ah, pl, o[2 * s + 1]);
    }
  }
};

// ---------------------------------------------------------------------------
// lengths and the deal of waves
// ---------------------------------------------------------------------------
// Keys of sample b: n buffer rows, the row of the new token (or -1), the
// first key of the window, and the new token's absolute position.
__device__ __forceinline__ void sample_keys(const DecodeParams& p, int b, int& n, int& newrow,
                                            int& kstart, int& last_pos) {
  if (p.len_mode == 0) n = p.lens[b] + 1;
  else if (p.len_mode == 1) n = p.lens[0] + 1;
  else if (p.len_mode == 3) n = p.lens[b];
  else n = p.host_n;
  last_pos = n - 1;
  // sliding-window cache: the buffer's rows after the eviction
  if (p.win_cap > 0) n = window_geom(n, 1, p.win_cap).fill;
  newrow = (p.k_new != nullptr) ? n - 1 : -1;
  if (n > p.cap) { n = p.cap; newrow = -1; }  // precondition violated: stay in bounds
  if (n < 0) { n = 0; newrow = -1; }
  kstart = (p.window >= 0) ? max(0, n - 1 - p.window) : 0;
}

// CSR block keys: entries [lo, hi) of layout l's column list for the row of
// the query at position n - 1 (clamped into the arrays, as for prompts).
__device__ __forceinline__ void csr_row(const DecodeParams& p, int l, int n, int& lo, int& hi) {
  lo = hi = 0;
  if (n <= 0) return;
  const int r = min((n - 1) / p.block, p.max_blocks - 1);
  lo = max(p.csr_rp[l * p.rp_stride + r], 0);
  hi = max(min(p.csr_rp[l * p.rp_stride + r + 1], (int)p.cols_stride), lo);
}

// Keys of the largest unit of a sample with n keys: every unit of the sample
// is dealt as many pairs (units of shorter rows get shorter runs).
__device__ int csr_max_keys(const DecodeParams& p, int n) {
  int m = 0;
  for (int l = 0; l < min(p.num_layout, p.N); ++l) {
    int lo, hi;
    csr_row(p, l, n, lo, hi);
    m = max(m, hi - lo);
  }
  return m * p.block;
}

template <bool CSR>
__device__ __forceinline__ int sample_count(const DecodeParams& p, int b) {
  int n, newrow, kstart, last_pos;
  sample_keys(p, b, n, newrow, kstart, last_pos);
  if constexpr (CSR) return csr_max_keys(p, n);
  return max(n - kstart, 0);
}

// Keys per pair of waves: every unit gets ceil(c / quota) pairs (at least
// one), with quota = max(128, ceil(K / (P - U))) for K live keys over U units
// and P = W / 2 pairs, so the units never need more than P pairs.  Called by
// all lanes of a wave; c0 is the count of sample `lane` (0 beyond the batch).
template <bool CSR>
__device__ int64_t deal_quota(const DecodeParams& p, int ups, int lane, int c0) {
  int64_t k = c0;
  for (int b = lane + 64; b < p.B; b += 64) k += sample_count<CSR>(p, b);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) k += __shfl_xor(k, m, 64);
  k *= ups;
  const int64_t units = (int64_t)p.B * ups;
  const int64_t spare = (int64_t)(p.waves / 2) - units;
  if (spare <= 0 || !p.split) return INT64_MAX;
  return max(2 * kMinKeysPerWave, (k + spare - 1) / spare);
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int pairs_for(int c, int64_t quota) {
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

// Sample served by pair pr and the first pair of that sample's units; false
// when pr is beyond the pairs in use.
template <bool CSR>
__device__ bool find_sample(const DecodeParams& p, int ups, int64_t quota, int pr, int lane, int c0,
                            int& b_out, int& first_out) {
  int base = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int b = b0 + lane;
    const int c = b0 == 0 ? c0 : (b < p.B ? sample_count<CSR>(p, b) : 0);
    const int v = (b < p.B) ? pairs_for(c, quota) * ups : 0;
    const int incl = wave_scan(v, lane);
    const bool hit = b < p.B && pr >= base + incl - v && pr < base + incl;
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

// Partial records merged per batch by the last pair of a unit (a unit split
// over at most this many pairs is merged after one round trip).
constexpr int kMergeBatch = 16;

// Partial records cross compute units on different XCDs, whose L2 caches are
// not coherent with each other: they are stored and loaded at device scope
// (the sc1 cache policy: written through to, and read from, the level all
// XCDs share), through a buffer resource over the partial records
// (out-of-range accesses read 0 and drop the store).
constexpr int kDeviceScope = 16;               // cache-policy bit of sc1
constexpr int kBufferFormat = 0x00020000;      // raw 32-bit buffer (gfx9 family)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const DecodeParams& p, int rs) {
  const int64_t bytes = (int64_t)(p.waves / 2) * p.hpw * rs * 4;
  return __builtin_amdgcn_make_buffer_rsrc(p.part, 0, (int)min(bytes, (int64_t)0x7fffffff), kBufferFormat);
}
__device__ __forceinline__ void store_partial_ml(__amdgpu_buffer_rsrc_t r, int off, float m, float l) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uint2v, float2v{m, l}), r, off, 0, kDeviceScope);
}
__device__ __forceinline__ void store_partial_o(__amdgpu_buffer_rsrc_t r, int off, float4v o) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint4v, o), r, off, 0, kDeviceScope);
}
__device__ __forceinline__ float2v load_partial_ml(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float2v, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kDeviceScope));
}
__device__ __forceinline__ float4v load_partial_o(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float4v, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDeviceScope));
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

// Calls f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>) in order.
template <typename F, int... Is>
__device__ __forceinline__ void static_for(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}

// As static_for, while f returns true.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_while(F&& f, std::integer_sequence<int, Is...>) {
  bool go = true;
  ((go = go && f(std::integral_constant<int, Is>{})), ...);
}

// FEAT bits: kSoftcap (scores are soft-capped), kExtras (additive bias and/or
// mask, and/or the qk output).  The plain variant has no per-score checks.
// kCsrKeys: keys are CSR blocks (SparseAttention token generation).
constexpr int kSoftcap = 1, kExtras = 2, kCsrKeys = 4;

template <typename T, int HP, int FEAT>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(DecodeParams p) {
  // the bias/mask/qk variant keeps one buffer less (more live state per score)
  constexpr int R = (FEAT & kExtras) ? (Ring<T, HP>::value > 1 ? Ring<T, HP>::value - 1 : 1)
                                     : Ring<T, HP>::value;
  using Tile = DecTile<T, HP, R>;
  using AT = typename ActOf<T>::type;    // query, new rows, rotary, bias, sink, output
  using CT = typename CacheOf<T>::type;  // cache elements
  constexpr bool kQ4 = std::is_same<T, QuantI4>::value;
  constexpr bool kQuant = std::is_same<T, QuantI8>::value || kQ4;
  using Q4 = Quad<AT>;
  using QT = typename Q4::type;
  constexpr int NQ = HP / 16, NH = NQ / 2;
  constexpr int RS = HP + 4;  // partial record: m, l, -, -, o[HP]
  __shared__ int s_claim[kPairsPerGroup];
  __shared__ __attribute__((aligned(16))) float s_part[kPartFloats];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int jp = wave % kPairsPerGroup;      // pair of this wave (waves jp, jp + 4 share a SIMD)
  const int younger = wave / kPairsPerGroup;
  const int pr = blockIdx.x * kPairsPerGroup + jp;
  if (tid < kPairsPerGroup) s_claim[tid] = 0;
  __syncthreads();

  const int H = p.H;
  const int g = p.N / p.kvN;
  const int hg = p.head_groups;
  const int ups = p.kvN * hg;

  // ---- which unit and which run of its keys (the same for both waves) -------
  // lane i reads the length of sample i once; the deal and this pair's sample
  // take it from there
  constexpr bool csr = (FEAT & kCsrKeys) != 0;  // p.csr_rp is set exactly then
  int n_l = 0, newrow_l = -1, kstart_l = 0, last_l = 0, c_l = 0;
  if (lane < p.B) {
    sample_keys(p, lane, n_l, newrow_l, kstart_l, last_l);
    c_l = csr ? csr_max_keys(p, n_l) : max(n_l - kstart_l, 0);
  }
  // (the deal is the same in every lane: the values are made scalar, so that
  // the chunk bookkeeping of the streaming loop runs on the scalar unit)
  const int64_t quota = uniform64(deal_quota<csr>(p, ups, lane, c_l));
  int b = 0, first = 0;
  const bool live = find_sample<csr>(p, ups, quota, pr, lane, c_l, b, first);
  b = __builtin_amdgcn_readfirstlane(b);
  first = __builtin_amdgcn_readfirstlane(first);
  int n = 0, newrow = -1, kstart = 0, last_pos = 0;
  if (b < 64) {
    n = __shfl(n_l, b, 64);
    newrow = __shfl(newrow_l, b, 64);
    kstart = __shfl(kstart_l, b, 64);
    last_pos = __shfl(last_l, b, 64);
  } else {
    sample_keys(p, b, n, newrow, kstart, last_pos);
  }
  n = __builtin_amdgcn_readfirstlane(n);
  newrow = __builtin_amdgcn_readfirstlane(newrow);
  kstart = __builtin_amdgcn_readfirstlane(kstart);
  last_pos = __builtin_amdgcn_readfirstlane(last_pos);
  int c_s = csr ? (b < 64 ? __shfl(c_l, b, 64) : csr_max_keys(p, n)) : max(n - kstart, 0);
  c_s = __builtin_amdgcn_readfirstlane(c_s);
  const int c = live ? c_s : 0;
  const int nb = pairs_for(c, quota);
  const int local = pr - first;
  const int ui = live ? local / nb : 0;
  const int kp = live ? local % nb : 0;  // pair within the unit
  const bool direct = nb == 1;  // the unit's only pair writes its output
  const int kvh = ui / hg, hgrp = ui % hg;
  const int h0 = kvh * g + hgrp * 16;
  const int nh = min(16, g - hgrp * 16);
  // the run [lo, lo + len) of the unit's keys; CSR units count their keys
  // block by block in row order ("virtual" keys) and cut runs at multiples of
  // 16, so that no 16-key sub-tile straddles two blocks
  int lo, len, csr_lo = 0;
  if constexpr (csr) {
    int e_hi;
    csr_row(p, kvh % p.num_layout, n, csr_lo, e_hi);
    csr_lo = __builtin_amdgcn_readfirstlane(csr_lo);
    const int cu = live ? __builtin_amdgcn_readfirstlane((e_hi - csr_lo) * p.block) : 0;
    lo = (int)((int64_t)cu * kp / nb) & ~15;
    const int hi = (kp == nb - 1) ? cu : ((int)((int64_t)cu * (kp + 1) / nb) & ~15);
    len = hi - lo;
  } else {
    lo = kstart + (int)((int64_t)c * kp / nb);
    len = kstart + (int)((int64_t)c * (kp + 1) / nb) - lo;
  }
  // chunks of the run: chunk ch holds keys [chunk_lo(ch), chunk_lo(ch + 1))
  // each pair owns a fixed slice of the LDS records: chunk ch, head hj at
  // pair_part + (ch * nh + hj) * RS (pairs of one group may differ in nh); a
  // CSR pair keeps the cache blocks of its run at the end of its slice
  constexpr int kSlice = kPartFloats / kPairsPerGroup;
  float* pair_part = s_part + jp * kSlice;
  const int blk0 = csr ? lo / p.block : 0;
  const int tbl_n = (csr && len > 0) ? (lo + len - 1) / p.block - blk0 + 1 : 0;
  int* tbl = reinterpret_cast<int*>(pair_part + kSlice) - tbl_n;
  const int nch_cap = max(1, min(kMaxChunks, (kSlice - tbl_n) / (nh * RS)));
  // chunks of csz keys (a multiple of 16, at least 32); the last may be short
  const int csz = len > 0 ? max(32, (len + nch_cap * 16 - 1) / (nch_cap * 16) * 16) : 32;
  const int nch = (len + csz - 1) / csz;
  // the new token's row is the unit's last key: the last chunk of its last
  // pair, kept for the older wave, which appends the row before reading it
  const bool append = live && newrow >= lo && newrow < lo + len;
  const bool appender = append && !younger;
  const int claimable = nch - (append ? 1 : 0);

  const int kv_div = csr ? max(p.kv_div, 1) : 1;
  const int64_t slab = (int64_t)b * (p.kvN / kv_div) + kvh / kv_div;
  const int rowel = kQ4 ? H / 2 : H;  // cache elements per row
  CT* kb = static_cast<CT*>(p.kc) + slab * p.cap * rowel;
  CT* vb = static_cast<CT*>(p.vc) + slab * p.cap * rowel;
  // CSR: the cache block of each block of the run (both waves of the pair
  // fill the table; every wave of the group passes the barrier)
  if constexpr (csr) {
    const int* cols = p.csr_cols + (int64_t)(kvh % p.num_layout) * p.cols_stride + csr_lo + blk0;
    for (int i = younger * 64 + lane; i < tbl_n; i += 128) tbl[i] = min(max(cols[i], 0), p.max_blocks - 1);
    __syncthreads();
  }
  const int half = H / 2;
  const AT* cs = static_cast<const AT*>(p.cos);
  const AT* sn = static_cast<const AT*>(p.sin);
  const bool rot = cs != nullptr;
  // rotary row of the new token: its absolute position (the last buffer row
  // unless a sliding-window cache has evicted rows)
  const int pos = min(max(last_pos, 0), max(p.rot_rows - 1, 0));
  const AT* cs_row = rot ? cs + (int64_t)pos * half : nullptr;
  const AT* sn_row = rot ? sn + (int64_t)pos * half : nullptr;

  // ---- the query: RMSNorm and rotary in registers ------------------------------
  // x[qi][e] = query element quad_dim(qi, g4) + e of head h0 + hh.  With H
  // equal to the padded size both members of a rotary pair (d, d + H/2) are
  // quads qi and qi + NQ/2 of the same lane, and the loads of the query, the
  // rotary rows and the appended row all go out together; other head sizes
  // load the partner quads.
  const int hh = lane & 15, g4 = lane >> 4;
  Tile tile;  // (the int8 tile's dims per quad depend on the head size)
  if constexpr (kQuant) tile.set_layout(H, lane);
  const AT* qrow = static_cast<const AT*>(p.q) + ((int64_t)b * p.N + h0 + min(hh, nh - 1)) * H;
  const AT* qw = static_cast<const AT*>(p.q_norm);
  const bool same_lane_pairs = (H == HP);
  float x[NQ][4];
  auto load_quads = [&](QT (&dst)[NQ], const AT* src, bool on) {
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi) {
      const int d = tile.quad_dim(qi, g4);
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
  // int8 caches: the key scales of the query's dims
  QT ksr[NQ];
  if constexpr (kQuant) {
    if (p.k_scale_pc) {
      load_quads(ksr, p.k_scale + (int64_t)kvh * H, true);
    } else {
      const float s0 = p.k_scale[0];
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) ksr[qi] = QT{s0, s0, s0, s0};
    }
  }
  if (same_lane_pairs) {
    load_quads(qr, qrow, true);
    load_quads(wr, qw, qw != nullptr);
    if (rot) {
#pragma unroll
      for (int qi = 0; qi < NH; ++qi) {
        const int d = tile.quad_dim(qi, g4);  // < H / 2
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
        const int d = tile.quad_dim(qi, g4);
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
  QT aks = Q4::zero(), avs = Q4::zero();  // int8 caches: scales of the row's dims
  if (append && alane) {
    const int64_t nrow = ((int64_t)b * p.kvN + kvh) * H;
    ak = Q4::load(static_cast<const AT*>(p.k_new) + nrow + ad);
    av = Q4::load(static_cast<const AT*>(p.v_new) + nrow + ad);
    if constexpr (kQuant) {
      if (p.k_scale_pc) aks = Q4::load(p.k_scale + (int64_t)kvh * H + ad);
      else aks = QT{p.k_scale[0], p.k_scale[0], p.k_scale[0], p.k_scale[0]};
      if (p.v_scale_pc) avs = Q4::load(p.v_scale + (int64_t)kvh * H + ad);
      else avs = QT{p.v_scale[0], p.v_scale[0], p.v_scale[0], p.v_scale[0]};
    }
    if (p.k_norm != nullptr) aw = Q4::load(static_cast<const AT*>(p.k_norm) + ad);
    if (rot) {
      const int i = ad < half ? ad : ad - half;
      ac = Q4::load(cs_row + i);
      as = Q4::load(sn_row + i);
    }
  }
  auto do_append = [&]() {
    pin(ak);
    pin(av);
    pin(aw);
    pin(ac);
    pin(as);
    if constexpr (kQuant) {
      pin(aks);
      pin(avs);
    }
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
      if constexpr (kQ4) {
        // dims 4l .. 4l + 3 are bytes 2l, 2l + 1 (even dim in the low nibble)
        uint32_t kw = 0, vw = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kw |= quant4(y[e], aks[e]) << (4 * e);
          vw |= quant4(av[e], avs[e]) << (4 * e);
        }
        *reinterpret_cast<uint16_t*>(kb + (int64_t)newrow * rowel + 2 * lane) = (uint16_t)kw;
        *reinterpret_cast<uint16_t*>(vb + (int64_t)newrow * rowel + 2 * lane) = (uint16_t)vw;
      } else if constexpr (kQuant) {
        uint32_t kw = 0, vw = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kw |= quant8(y[e], aks[e]) << (8 * e);
          vw |= quant8(av[e], avs[e]) << (8 * e);
        }
        *reinterpret_cast<uint32_t*>(kb + (int64_t)newrow * H + ad) = kw;
        *reinterpret_cast<uint32_t*>(vb + (int64_t)newrow * H + ad) = vw;
      } else {
        Q4::store(kb + (int64_t)newrow * H + ad, y);
        Q4::store_raw(vb + (int64_t)newrow * H + ad, av);
      }
    }
    // The row is read back by other lanes of this wave: order the stores
    // before those loads (no instruction is needed within one wave).  The
    // stores are also retired here: loads and stores share one counter, and
    // a store left pending past the join would make every later wait of the
    // other waves a full drain.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  };

  // ---- streaming: chunks claimed by the two waves of the pair ----------------
  // Chunk sub-tiles go through a ring of R register buffers; the load of the
  // sub-tile R - 1 places ahead is issued before a sub-tile is computed, and
  // the next chunk is claimed when the loads reach the end of the current one.
  // Loads are issued on every step (past the end they re-read a valid row), so
  // every path between a load and its use issues the same loads.
  auto claim = [&]() -> int {
    int v = 0;
    if (lane == 0) v = atomicAdd(&s_claim[jp], 1);
    v = __builtin_amdgcn_readfirstlane(__shfl(v, 0, 64));
    return v < claimable ? v : nch;
  };
  // next load: chunk lc, its keys [ca, ce), sub-tile ls of ns
  int lc = nch, ls = 0, ca = 0, ce = 0, ns = 0;
  auto enter = [&](int ch) {
    lc = ch;
    ls = 0;
    ca = lo + ch * csz;
    ce = min(ca + csz, lo + len);
    ns = (ce - ca + 15) / 16;
  };
  if (live) enter(appender ? nch - 1 : claim());
  // b_off: cache row minus key index in the sub-tile (CSR block keys; else 0)
  int b_j0[R], b_end[R], b_ch[R], b_off[R];
  bool b_last[R];
  auto next_load = [&](auto rt) {
    constexpr int r = decltype(rt)::value;
    b_off[r] = 0;
    if (lc < nch) {
      b_j0[r] = ca + 16 * ls;
      b_end[r] = ce;
      b_ch[r] = lc;
      b_last[r] = ls == ns - 1;
      if constexpr (csr) {
        const int e = b_j0[r] / p.block;
        b_off[r] = __builtin_amdgcn_readfirstlane((tbl[e - blk0] - e) * p.block);
      }
      if (++ls == ns) enter(claim());
    } else {
      b_j0[r] = kstart;
      b_end[r] = kstart + 1;
      b_ch[r] = -1;
      b_last[r] = false;
    }
    // rows of the sub-tile (a 16-key sub-tile lies inside one block)
    const int pj = min(b_j0[r] + b_off[r], p.cap - 1);
    const int pl = min(min(b_end[r] - 1, b_j0[r] + 15) + b_off[r], p.cap - 1);
    tile.template load_kv<r>(kb, vb, pj, pl, H, lane);
  };
  // ---- finish the query (and the append) before streaming --------------------
  // The query and rotary rows are isolated lines: issued behind the key/value
  // stream of the whole grid they would wait for most of it, so every wave
  // completes them while the memory system is still idle.
  if (appender) do_append();
  tile.init();
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
  // int8 caches: fold the key scales into the query and bring the head's
  // largest |element| into [2^13, 2^14) (scores are scaled back in smul)
  float smul = p.scale;
  if constexpr (kQuant) {
    float mx = 0.f;
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[qi][e] *= ksr[qi][e];
        mx = fmaxf(mx, fabsf(x[qi][e]));
      }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    int ex = 0;
    frexpf(mx, &ex);
    const int sh = min(max(14 - ex, -60), 60);
    const float up = ldexpf(1.f, sh);
#pragma unroll
    for (int qi = 0; qi < NQ; ++qi)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[qi][e] *= up;
    smul = p.scale * ldexpf(1.f, -sh);
  }
  tile.set_q(x);

  // identity for the f16 V transpose: lane l holds B[k = 4(l/16)+i][n = l%16]
  half4v ident;
#pragma unroll
  for (int i = 0; i < 4; ++i) ident[i] = (f16)((4 * g4 + i) == hh ? 1.f : 0.f);

  const bool head_ok = hh < nh;
  const int h = h0 + hh;
  const float cap = p.softcap, inv_cap = p.softcap > 0.f ? 1.f / p.softcap : 0.f;
  const AT* bias = static_cast<const AT*>(p.bias);
  void* const qk = p.qk;

  float m = kNegInf, l = 0.f;
  // plain scores go to the log2 domain in the same multiply
  const float smul_l2 = smul * kLog2e;
  // Score transform, online softmax and PV for the sub-tile held in BUF.
  // The running max m moves only when a score exceeds it by more than
  // kDecodeSlack (log2 units): the probabilities then stay <= 2^kDecodeSlack
  // and the rescale of the output is skipped on most sub-tiles.
  auto process = [&](auto buf_tag, int j0, int j_end) {
    constexpr int BUF = decltype(buf_tag)::value;
    const float4v sc = tile.template scores<BUF>();
    mfma_result_fence();
    float tmax = kNegInf;
    float4v x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = j0 + 4 * g4 + i;
      const bool ok = head_ok && key < j_end;
      if constexpr ((FEAT & (kSoftcap | kExtras)) == 0) {
        const float v = sc[i] * smul_l2;
        x[i] = ok ? v : kNegInf;
        tmax = fmaxf(tmax, x[i]);
        continue;
      }
      float v = sc[i] * smul;
      if (FEAT & kSoftcap) v = softcap_apply(v, cap, inv_cap);
      if (FEAT & kExtras) {
        if (ok && bias != nullptr && key < p.bias_cols)
          v += to_f32(bias[b * p.bias_sb + h * p.bias_sh + key]);
        if (ok && p.mask != nullptr && key < p.mask_cols)
          v += (p.mask[(int64_t)b * p.mask_cols + key] == 0) ? p.mask_filter : 0.f;
        if (ok && qk != nullptr) {
          const int64_t at = ((int64_t)b * p.N + h) * p.host_n + key;
          if (p.qk_f32) static_cast<float*>(qk)[at] = v;
          else static_cast<f16*>(qk)[at] = from_f32<f16>(v);
        }
      }
      v = ok ? v * kLog2e : kNegInf;
      x[i] = v;
      tmax = fmaxf(tmax, v);
    }
    tmax = fmaxf(tmax, shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const bool grow = tmax > m + kDecodeSlack;
    if (__any(grow)) {
      // a side effect keeps this a branch (executed unconditionally the
      // rescale would cost a multiply per accumulator on every sub-tile)
      asm volatile("" ::: "memory");
      const float alpha = grow ? fast_exp2(m - tmax) : 1.f;
      m = grow ? tmax : m;
      l *= alpha;
      tile.scale_o(alpha);
    }
    const float muse = (m == kNegInf) ? 0.f : m;
    float4v pr;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = fast_exp2(x[i] - muse);
      pr[i] = e;
      psum += e;
    }
    l += psum;
    tile.template pv<BUF>(pr, ident);
  };

  // the chunk's (m, l, o) into its LDS record; the state restarts
  auto flush = [&](int ch) {
    mfma_result_fence();
    const float lt = l + shfl_xor(l, 16) + shfl_xor(l, 32) + shfl_xor(shfl_xor(l, 16), 32);
    if (head_ok) {
      float* row = pair_part + (ch * nh + hh) * RS;
      if (g4 == 0) *reinterpret_cast<float2v*>(row) = float2v{m, lt};
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) {
        const int d = tile.quad_dim(qi, g4);
        if (d < H) *reinterpret_cast<float4v*>(row + 4 + d) = tile.o[qi];
      }
    }
    m = kNegInf;
    l = 0.f;
    tile.init();
  };
  static_for(next_load, std::make_integer_sequence<int, R - 1>{});
  bool go = live;
  while (go) {
    static_for(
        [&](auto rt) {
          constexpr int r = decltype(rt)::value;
          next_load(std::integral_constant<int, (r + R - 1) % R>{});
          if (go && b_ch[r] >= 0) {
            // CSR block keys: visible up to the query's own row
            const int j_end = csr ? min(b_end[r], last_pos - b_off[r] + 1) : b_end[r];
            process(std::integral_constant<int, r>{}, b_j0[r], j_end);
            if (b_last[r]) flush(b_ch[r]);
          } else {
            go = false;
          }
        },
        std::make_integer_sequence<int, R>{});
  }
  mfma_result_fence();
  __syncthreads();

  // ---- merge the pair's chunks in chunk order: output or the pair's partial --
  const int t = younger * 64 + lane;
  constexpr int NQD = HP / 4;
  const __amdgpu_buffer_rsrc_t part = partial_rsrc(p, RS);
  if (live) {
    for (int e = t; e < nh * NQD; e += 2 * 64) {
      const int hj = e / NQD, d = 4 * (e % NQD);
      if (d >= H) continue;
      const float* base = pair_part + hj * RS;
      float M = kNegInf;
      for (int ch = 0; ch < nch; ++ch) M = fmaxf(M, base[ch * nh * RS]);
      const float Mu = (M == kNegInf) ? 0.f : M;
      float L = 0.f;
      float4v O = {0.f, 0.f, 0.f, 0.f};
      for (int ch = 0; ch < nch; ++ch) {
        const float* row = base + ch * nh * RS;
        const float f = fast_exp2(row[0] - Mu);
        L += row[1] * f;
        O += *reinterpret_cast<const float4v*>(row + 4 + d) * f;
      }
      const int hq = h0 + hj;
      if constexpr (kQuant) {
        // value scales, and the 2^12 of the probabilities
        const float u = 1.f / Tile::kPScale;
        if (p.v_scale_pc) O *= *reinterpret_cast<const float4v*>(p.v_scale + (int64_t)kvh * H + d) * u;
        else O *= p.v_scale[0] * u;
      }
      if (direct) {
        bool has;
        const float sg = read_sink<AT>(p, hq, has);
        const float inv = final_scale(M, L, has, sg);
        const float v[4] = {O[0] * inv, O[1] * inv, O[2] * inv, O[3] * inv};
        Q4::store(static_cast<AT*>(p.out) + ((int64_t)b * p.N + hq) * H + d, v);
      } else {
        const int rec = ((pr * p.hpw + hj) * RS) * 4;  // byte offset of the record
        if (d == 0) store_partial_ml(part, rec, M, L);
        store_partial_o(part, rec + (4 + d) * 4, O);
      }
    }
  }

  // ---- arrival: the last pair of a split unit merges the unit's partials ------
  // The partials are written through to the device-coherent level (no L2
  // write-back of the whole cache is needed); each wave waits for its stores
  // to complete before the group barrier, then one lane per pair counts the
  // pair in.  The counter goes back to zero when the unit is merged, so the
  // next call finds it so.
  __shared__ int s_last[kPairsPerGroup];
  const bool split = live && !direct;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's partial stores are done
  __syncthreads();
  const int unit = b * ups + ui;
  if (!younger && lane == 0) {
    int last = 0;
    if (split)
      last = __hip_atomic_fetch_add(p.counters + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nb - 1;
    s_last[jp] = last;
  }
  __syncthreads();
  if (!s_last[jp]) return;
  const int pair0 = first + ui * nb;
  const int rstride = p.hpw * RS * 4;  // bytes between the unit's pair records
  for (int e = t; e < nh * NQD; e += 2 * 64) {
    const int hj = e / NQD, d = 4 * (e % NQD);
    if (d >= H) continue;
    const int base = ((pair0 * p.hpw + hj) * RS) * 4;
    const int hq = h0 + hj;
    // the sink's load is in flight with the first batch
    bool has;
    const float sg = read_sink<AT>(p, hq, has);
    // records in batches of kMergeBatch, all loads of a batch in flight at
    // once (each is a round trip to the shared level); the running (M, L, O)
    // is rescaled once per batch
    float M = kNegInf, L = 0.f;
    float4v O = {0.f, 0.f, 0.f, 0.f};
    for (int i0 = 0; i0 < nb; i0 += kMergeBatch) {
      float2v mlb[kMergeBatch];
      float4v ob[kMergeBatch];
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        const int rec = base + min(i0 + k, nb - 1) * rstride;
        mlb[k] = load_partial_ml(part, rec);
        ob[k] = load_partial_o(part, rec + (4 + d) * 4);
      }
      float mn = M;
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k)
        if (i0 + k < nb) mn = fmaxf(mn, mlb[k][0]);
      const float mu = (mn == kNegInf) ? 0.f : mn;
      const float fo = fast_exp2(M - mu);
      L *= fo;
      O *= fo;
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k)
        if (i0 + k < nb) {
          const float f = fast_exp2(mlb[k][0] - mu);
          L += mlb[k][1] * f;
          O += ob[k] * f;
        }
      M = mn;
    }
    const float inv = final_scale(M, L, has, sg);
    const float v[4] = {O[0] * inv, O[1] * inv, O[2] * inv, O[3] * inv};
    Q4::store(static_cast<AT*>(p.out) + ((int64_t)b * p.N + hq) * H + d, v);
  }
  if (t == 0) __hip_atomic_store(p.counters + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int HP, int FEAT>
hipError_t launch_decode_f(const DecodeParams& p, hipStream_t s) {
  launch_kernel((decode_kernel<T, HP, FEAT>), dim3(p.waves / kWavesPerGroup), dim3(kThreads),
                     0, s, p);
  return hipGetLastError();
}

template <typename T, int HP>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
  if constexpr (!std::is_same<T, QuantI8>::value && !std::is_same<T, QuantI4>::value) {
    // CSR block keys come without bias, mask, qk or softcap
    if (p.csr_rp != nullptr) return launch_decode_f<T, HP, kCsrKeys>(p, s);
  }
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
  if (p.B == 0) return hipSuccess;
  if (dt == DType::F16) {
    if (hp == 64) return launch_decode_t<f16, 64>(p, s);
    if (hp == 128) return launch_decode_t<f16, 128>(p, s);
    return launch_decode_t<f16, 256>(p, s);
  }
  if (dt == DType::Q8) {
    if (hp == 64) return launch_decode_t<QuantI8, 64>(p, s);
    if (hp == 128) return launch_decode_t<QuantI8, 128>(p, s);
    return launch_decode_t<QuantI8, 256>(p, s);
  }
  if (dt == DType::Q4) {
    if (hp == 64) return launch_decode_t<QuantI4, 64>(p, s);
    if (hp == 128) return launch_decode_t<QuantI4, 128>(p, s);
    return launch_decode_t<QuantI4, 256>(p, s);
  }
  if (hp == 64) return launch_decode_t<float, 64>(p, s);
  if (hp == 128) return launch_decode_t<float, 128>(p, s);
  return launch_decode_t<float, 256>(p, s);
}

}  // namespace kvattn
