// K2: tiled online-softmax attention on MFMA (prefill / prompt paths).
//
// A work item is a block of query rows for one or more query heads that
// share a kv head; every wave owns 32 query rows of one head.  Key/value
// tiles of BN rows are staged in LDS and shared by the waves of the item:
// flash_pp_kernel (dense f16 prompts, heads up to 128) copies them
// from global memory straight into LDS and runs two items per workgroup in
// alternating MFMA and softmax phases; flash_kernel (block-sparse, varlen,
// float32, heads of 256) fills double-buffered LDS tiles from registers
// loaded one tile ahead.
//
//   S^T[keys][32 queries] = K_tile . Q^T        (f16: 32x32x16, f32: 32x32x2)
//   O^T[H][32 queries]   += V_tile^T . P^T
//
// With the scores transposed, each lane holds one query's scores, so the
// running max/sum (online softmax) needs one cross-lane step (lane ^ 32) per
// tile, and P^T leaves the score MFMA already in the operand layout of the
// PV MFMA (the contraction order over keys is permuted to match).  For f16
// the V^T operand is read from the row-major LDS tile with ds_read_b64_tr_b16.
//
// Modes (one kernel template):
//   dense  - GroupQueryAttention: causal bound right-aligned to the live
//            length (seqlens_k), optional local window, softcap, additive bias,
//            head sink / smooth softmax, or bidirectional without a past
//            (GroupQueryAttention page: Inputs and Attributes tables;
//            Implementation variants on causal tile skipping).
//   csr    - SparseAttention: the key tiles of a query block come from its CSR
//            row (layout = head mod num_layout), causal inside the diagonal
//            block (SparseAttention page: Description and Inputs table).
//   varlen - PackedAttention: each token attends the keys of its own
//            sequence [cum[b], cum[b+1]); work items come from a device work
//            list (PackedAttention page: Description and Inputs table).
#include <type_traits>
#include <utility>

#include "device_common.hpp"
#include "kvattn_internal.hpp"

namespace kvattn {
namespace {

typedef __fp16 lds_half4 __attribute__((__vector_size__(4 * sizeof(__fp16))));

// instruction classes of sched_group_barrier masks
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedDsRead = 0x100;
// s_waitcnt operand: vmcnt(0), other counters unconstrained
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ __forceinline__ half4v lds_read_tr16(const f16* p) {
  auto r = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (__attribute__((address_space(3))) lds_half4*)(p));
  half4v o;
  o[0] = (f16)r[0];
  o[1] = (f16)r[1];
  o[2] = (f16)r[2];
  o[3] = (f16)r[3];
  return o;
}

template <typename T, int HP> struct FlashMma;

// ------------------------------- f16 ----------------------------------------
template <int HP> struct FlashMma<f16, HP> {
  static constexpr int KS = HP + 8;    // K tile row stride (elements): rows 4 banks apart
  // V tile row stride (elements): 32 or 96 modulo 128, so that the two
  // 16-lane groups of a transposing read hit disjoint bank halves
  static constexpr int VS = HP <= 64 ? 96 : (HP <= 128 ? 160 : 288);
  static constexpr int NS = HP / 16;   // 16-dim k-steps of the score MFMA
  static constexpr int ND = HP / 32;   // 32-dim output blocks
  static constexpr int CH = 8;         // elements per 16-byte chunk
  static constexpr int NE = HP / 2;    // query elements per lane
  static constexpr bool kPairInLane = true;  // interleaved rotary pairs share a lane
  half8v qf[NS];
  float16v o[ND];

  __device__ void init() {
#pragma unroll
    for (int i = 0; i < ND; ++i) o[i] = float16v{};
  }
  // lane l holds Q[q = l%32][edim(e, l/32)], e < NE
  __device__ static int edim(int e, int h) { return 16 * (e >> 3) + 8 * h + (e & 7); }
  __device__ static void load_raw(const f16* qrow, int H, int lane, float (&x)[NE]) {
    const int h = lane >> 5;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int d = 16 * s + 8 * h;
      const half8v v = (d < H) ? load_half8(qrow + d) : half8v{};
#pragma unroll
      for (int i = 0; i < 8; ++i) x[8 * s + i] = (float)v[i];
    }
  }
  // a row laid out like the query, unconverted: element e is r[e / 8][e % 8]
  // (NR = NS: all of it; NR = NS / 2: elements e < NE / 2, the first members
  // of the NeoX pairs)
  using Raw = half8v;
  template <int NR>
  __device__ static void load_rows(const f16* row, int H, int lane, Raw (&r)[NR]) {
    const int h = lane >> 5;
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      const int d = 16 * s + 8 * h;
      r[s] = (d < H) ? load_half8(row + d) : half8v{};
    }
  }
  __device__ static float raw_at(const Raw* r, int e) { return (float)r[e >> 3][e & 7]; }
  static constexpr int kRawPer = 8;   // elements per Raw
  __device__ void set_q(const float (&x)[NE]) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      half8v v;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (f16)x[8 * s + i];
      qf[s] = v;
    }
  }
  __device__ float16v qk_block(const f16* Kt, int kb, int lane) const {
    float16v acc = {};
    const f16* kr = Kt + (kb + (lane & 31)) * KS + 8 * (lane >> 5);
    // operand reads run one k-step ahead of the MFMA that uses them
    half8v a = *reinterpret_cast<const half8v*>(kr);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      half8v nxt = a;
      if (s + 1 < NS) nxt = *reinterpret_cast<const half8v*>(kr + 16 * (s + 1));
      acc = mfma32x32x16(a, qf[s], acc);
      a = nxt;
    }
    return acc;
  }
  // both 32-key blocks of a 64-key tile, interleaved, reads one step ahead
  // (PIN: fix the issue order of reads and MFMAs here; otherwise the caller does)
  template <bool PIN = true>
  __device__ void qk_tile64(const f16* Kt, int lane, float16v (&acc)[2]) const {
    acc[0] = float16v{};
    acc[1] = float16v{};
    const f16* k0 = Kt + (lane & 31) * KS + 8 * (lane >> 5);
    const f16* k1 = k0 + 32 * KS;
    half8v a0 = *reinterpret_cast<const half8v*>(k0);
    half8v a1 = *reinterpret_cast<const half8v*>(k1);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      half8v n0 = a0, n1 = a1;
      if (s + 1 < NS) {
        n0 = *reinterpret_cast<const half8v*>(k0 + 16 * (s + 1));
        n1 = *reinterpret_cast<const half8v*>(k1 + 16 * (s + 1));
      }
      acc[0] = mfma32x32x16(a0, qf[s], acc[0]);
      acc[1] = mfma32x32x16(a1, qf[s], acc[1]);
      a0 = n0;
      a1 = n1;
    }
    // issue order: four operand reads, then one MFMA and one read at a time,
    // so that each read is several MFMAs ahead of its use
    if (PIN) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * NS - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
    }
  }
  // both 32-key blocks of a 64-key tile (pb[2 * blk + half]: this lane's
  // probabilities of 16 keys each, in f16), operand reads pinned ahead of the
  // MFMAs that use them
  __device__ void pv_tile64(const f16* Vt, const half8v (&pb)[4], int lane) {
    const int G = lane >> 4, t = lane & 15;
    const int c = t & 3, ir = t >> 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // q = 2 * block + half: 16 keys each
      const int row = 16 * q + 4 * (G >> 1) + ir;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const f16* a1 = Vt + row * VS + 32 * db + 16 * (G & 1) + 4 * c;
        half4v lo = lds_read_tr16(a1);
        half4v hi = lds_read_tr16(a1 + 8 * VS);
        half8v a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[db] = mfma32x32x16(a, pb[q], o[db]);
      }
    }
    // six reads (three MFMAs' operands) ahead, then one MFMA and its
    // successor's two reads at a time
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 0);
#pragma unroll
    for (int i = 0; i < 4 * ND - 3; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 3, 0);
  }
  // p: this lane's 16 probabilities of the 32-key block at kb
  __device__ void pv_block(const f16* Vt, int kb, const float (&p)[16], int lane) {
    const int G = lane >> 4, t = lane & 15;
    const int c = t & 3, ir = t >> 2;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      half8v pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = (f16)p[8 * hf + i];
      const int row = kb + 16 * hf + 4 * (G >> 1) + ir;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const f16* a1 = Vt + row * VS + 32 * db + 16 * (G & 1) + 4 * c;
        half4v lo = lds_read_tr16(a1);
        half4v hi = lds_read_tr16(a1 + 8 * VS);
        half8v a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[db] = mfma32x32x16(a, pb, o[db]);
      }
    }
  }
};

// ------------------------------- f32 ----------------------------------------
template <int HP> struct FlashMma<float, HP> {
  static constexpr int KS = HP + 4;
  static constexpr int VS = HP + 4;
  static constexpr int NS = HP / 2;    // 2-dim k-steps of the score MFMA
  static constexpr int ND = HP / 32;
  static constexpr int CH = 4;
  static constexpr int NE = HP / 2;
  static constexpr bool kPairInLane = false;  // interleaved pairs: lanes l and l ^ 32
  float qf[NS];
  float16v o[ND];

  __device__ void init() {
#pragma unroll
    for (int i = 0; i < ND; ++i) o[i] = float16v{};
  }
  // lane l holds Q[q = l%32][edim(e, l/32)] = Q[q][2e + l/32]
  __device__ static int edim(int e, int h) { return 2 * e + h; }
  __device__ static void load_raw(const float* qrow, int H, int lane, float (&x)[NE]) {
    const int h = lane >> 5;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int d = 2 * s + h;
      x[s] = (d < H) ? qrow[d] : 0.f;
    }
  }
  using Raw = float;
  template <int NR>
  __device__ static void load_rows(const float* row, int H, int lane, Raw (&r)[NR]) {
    const int h = lane >> 5;
#pragma unroll
    for (int e = 0; e < NR; ++e) {
      const int d = 2 * e + h;
      r[e] = (d < H) ? row[d] : 0.f;
    }
  }
  __device__ static float raw_at(const Raw* r, int e) { return r[e]; }
  static constexpr int kRawPer = 1;
  __device__ void set_q(const float (&x)[NE]) {
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = x[s];
  }
  __device__ float16v qk_block(const float* Kt, int kb, int lane) const {
    float16v acc = {};
    const float* kr = Kt + (kb + (lane & 31)) * KS + (lane >> 5);
#pragma unroll
    for (int s = 0; s < NS; ++s) acc = mfma32x32x2f32(kr[2 * s], qf[s], acc);
    return acc;
  }
  __device__ void pv_block(const float* Vt, int kb, const float (&p)[16], int lane) {
    const int hi = lane >> 5, col = lane & 31;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int key = kb + 8 * (t >> 2) + 4 * hi + (t & 3);
      const float* vr = Vt + key * VS + col;
#pragma unroll
      for (int db = 0; db < ND; ++db) o[db] = mfma32x32x2f32(vr[32 * db], p[t], o[db]);
    }
  }
};

// Slack of the running maximum (log2 domain): see the online softmax below.
constexpr float kMaxSlack = 8.f;

// Tile schedule of one workgroup: tile t covers keys [start, start + BN) of
// which [start, lim) may be visible.
struct TileRange {
  int start, lim;
};

// The query row of this lane as the score MFMA operand: per-head RMSNorm
// (GroupQueryAttention page, Inputs table: q_norm_weight, before rotary),
// rotary at position pos (GroupQueryAttention page, Inputs table: cos/sin_cache;
// SparseAttention page, Attributes table: rotary_interleaved; the first
// 2 * rot_half dims rotate), then the factor qscale that turns the scores
// into the exponent the softmax needs.  Lanes l and l ^ 32 share a row.
// prep_query_issue sends every load of the row (query, norm weights, cos /
// sin) before any is used, so a row costs one memory latency;
// prep_query_finish does the arithmetic.
template <typename Mma> struct QueryLoads {
  static constexpr int NR = Mma::NE / Mma::kRawPer;
  typename Mma::Raw xr[NR], wr[NR], cr[NR / 2], sr[NR / 2];
};

// both members of every NeoX pair (d, d + H/2) are elements e, e + NE/2 of a lane
template <typename Mma>
__device__ __forceinline__ bool neox_in_lane(const FlashParams& p) {
  return p.cos != nullptr && !p.interleaved && 2 * p.rot_half == p.H && p.H == Mma::NE * 2;
}

template <typename Mma, typename T>
__device__ void prep_query_issue(QueryLoads<Mma>& ql, const T* qrow, int pos, const FlashParams& p, int lane) {
  const int H = p.H;
  const T* qn = static_cast<const T*>(p.q_norm);
  Mma::load_rows(qrow, H, lane, ql.xr);
  if (qn != nullptr) Mma::load_rows(qn, H, lane, ql.wr);
  if (neox_in_lane<Mma>(p)) {
    const int prow = min(max(pos, 0), p.rot_rows - 1);
    Mma::load_rows(static_cast<const T*>(p.cos) + (int64_t)prow * p.rot_half, H, lane, ql.cr);
    Mma::load_rows(static_cast<const T*>(p.sin) + (int64_t)prow * p.rot_half, H, lane, ql.sr);
  }
}

template <typename Mma, typename T>
__device__ void prep_query_finish(Mma& mma, const QueryLoads<Mma>& ql, const T* qrow, int pos,
                                  const FlashParams& p, float qscale, int lane) {
  constexpr int NE = Mma::NE;
  const int H = p.H, h = lane >> 5;
  const T* qn = static_cast<const T*>(p.q_norm);
  const T* cs = static_cast<const T*>(p.cos);
  const T* sn = static_cast<const T*>(p.sin);
  const int rh = p.rot_half;
  const int prow = min(max(pos, 0), p.rot_rows - 1);
  const T* cr = cs + (int64_t)prow * rh;
  const T* sr = sn + (int64_t)prow * rh;
  float x[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) x[e] = Mma::raw_at(ql.xr, e);
  float rn = 1.f;
  if (qn != nullptr) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) ss += x[e] * x[e];
    ss += shfl_xor(ss, 32);
    rn = rsqrtf(ss / (float)H + p.eps);
#pragma unroll
    for (int e = 0; e < NE; ++e) x[e] *= rn * Mma::raw_at(ql.wr, e);
  }
  if (neox_in_lane<Mma>(p)) {
#pragma unroll
    for (int e = 0; e < NE / 2; ++e) {
      const float c = Mma::raw_at(ql.cr, e), s = Mma::raw_at(ql.sr, e);
      const float a = x[e], z = x[e + NE / 2];
      x[e] = a * c - z * s;
      x[e + NE / 2] = z * c + a * s;
    }
  } else if (cs != nullptr) {
    if (p.interleaved) {
      // pairs (2i, 2i + 1): the partner is element e ^ 1 (f16) or lane l ^ 32 (f32)
      float y[NE];
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int d = Mma::edim(e, h);
        float z;
        if (Mma::kPairInLane) z = x[e ^ 1];
        else z = shfl_xor(x[e], 32);
        y[e] = x[e];
        if (d < 2 * rh) {
          const float c = to_f32(cr[d >> 1]), s = to_f32(sr[d >> 1]);
          y[e] = (d & 1) ? x[e] * c + z * s : x[e] * c - z * s;
        }
      }
#pragma unroll
      for (int e = 0; e < NE; ++e) x[e] = y[e];
    } else {
      // general NeoX width: the partner comes from memory (normed the same way)
      float y[NE];
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int d = Mma::edim(e, h);
        y[e] = x[e];
        if (d < 2 * rh && d < H) {
          const int pd = d < rh ? d + rh : d - rh;
          const int i = d < rh ? d : d - rh;
          float z = to_f32(qrow[pd]);
          if (qn != nullptr) z *= rn * to_f32(qn[pd]);
          const float c = to_f32(cr[i]), s = to_f32(sr[i]);
          y[e] = d < rh ? x[e] * c - z * s : x[e] * c + z * s;
        }
      }
#pragma unroll
      for (int e = 0; e < NE; ++e) x[e] = y[e];
    }
  }
#pragma unroll
  for (int e = 0; e < NE; ++e) x[e] *= qscale;
  mma.set_q(x);
}

template <typename Mma, typename T>
__device__ void prep_query(Mma& mma, const T* qrow, int pos, const FlashParams& p, float qscale,
                           int lane) {
  QueryLoads<Mma> ql;
  prep_query_issue<Mma>(ql, qrow, pos, p, lane);
  prep_query_finish(mma, ql, qrow, pos, p, qscale, lane);
}

// What one workgroup and wave of a flash launch cover: sample, heads, query
// rows, the key range and its tile schedule, and the K/V slab base.
template <int MODE, int BN> struct FlashWork {
  int b, kvh, h, r0, nrows;  // nrows: valid query rows of this workgroup's row block
  int wrow0, wg_rows_end;    // this wave's first row; end of the workgroup's rows
  bool wave_rows;            // the wave owns at least one valid row
  int n_keys, past, pmin, pmax, k_lo, k_hi;
  int rot_past;              // absolute position of query row 0 (rotary)
  int n_tiles, csr_lo, layout, tiles_per_block;
  int64_t row_base;          // varlen: first packed token of the sequence
  int64_t kv_base;           // K/V slab of (sample, kv head), in elements

  // false when the workgroup has no work item (varlen grids are padded)
  __device__ bool init(const FlashParams& p, int wave) {
    const int gx = gridDim.x, gy = gridDim.y, gz = gridDim.z;
    int id = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
    // Workgroups are dealt to the eight XCDs round-robin by linear id; the
    // remap gives each XCD a contiguous range of (row block, head group,
    // sample) items, so the workgroups sharing a K/V slab share one L2.
    if (MODE != kVarlen) id = xcd_grouped(id, gx * gy * gz);
    if (MODE == kCsr) id = csr_order(p, id, gx, gy);
    return init_item(p, wave, id, gx, gy, gz);
  }

  // Block-sparse prompts with one head per workgroup: the heads of one kv
  // head take the same group of kCsrRowGroup row blocks together (row block
  // fastest, then head, then row group, then kv head and sample), so the
  // K/V blocks in flight on an XCD are the local and vertical blocks of a
  // few dozen row blocks of one slab, which fit its L2.  Maps a position in
  // that order to the item id init_item expects.
  static constexpr int kCsrRowGroup = 16;
  __device__ static int csr_order(const FlashParams& p, int id, int gx, int gy) {
    const int g = p.N / p.kvN;
    if (p.heads_per_wg != 1 || gx % kCsrRowGroup != 0 || gy != p.N) return id;
    int t = id;
    const int r = t % kCsrRowGroup;
    t /= kCsrRowGroup;
    const int hh = t % g;
    t /= g;
    const int ng = gx / kCsrRowGroup;
    const int rg = t % ng;
    t /= ng;
    const int kvh = t % p.kvN;
    const int b = t / p.kvN;
    return (rg * kCsrRowGroup + r) + gx * ((kvh * g + hh) + gy * b);
  }

  // linear id -> id of a contiguous per-XCD range (n ids dealt round-robin
  // over eight XCDs)
  __device__ static int xcd_grouped(int id, int n) {
    return (n % 8 == 0) ? (id % 8) * (n / 8) + id / 8 : id;
  }

  // Work item `id` of a (gx, gy, gz) item grid (the layout of the launch grid
  // of the one-item-per-workgroup kernels).
  // lens: a copy of the first nlens entries of p.lens (dense mode), or null
  __device__ bool init_item(const FlashParams& p, int wave, int id, int gx, int gy, int gz,
                            const int* lens = nullptr, int nlens = 0) {
    const int g = p.N / p.kvN;
    const int HW = p.heads_per_wg;
    row_base = 0;
    if (MODE == kVarlen) {
      // item-major: all heads of the list's first (longest) item go first
      const int count = p.work[0];
      const int item = id / gy;
      if (item >= count) return false;
      b = p.work[1 + 2 * item];
      const int tile = p.work[2 + 2 * item];
      h = id % gy;
      kvh = h / g;
      r0 = tile * p.rows_per_wg;
      row_base = p.lens[2 * b];
      nrows = p.lens[2 * b + 1] - p.lens[2 * b];
    } else {
      // Row blocks go last to first: under a causal bound the late blocks see
      // the most keys, so the longest items start first and short ones fill
      // the tail.
      if (id >= gx * gy * gz) return false;
      const int bx = gx - 1 - id % gx, by = (id / gx) % gy;
      b = id / (gx * gy);
      const int groups = g / HW;
      kvh = by / groups;
      h = kvh * g + (by % groups) * HW + (wave % HW);
      r0 = bx * p.rows_per_wg;
      nrows = p.S;
      // CSR token generation: a workgroup's rows are one block of absolute
      // positions (one CSR row), so the blocks start (past mod block) rows
      // early and the grid has one workgroup more; rows before 0 do not exist
      if (MODE == kCsr && p.has_past) {
        r0 -= max(p.key_total[b] - p.S, 0) % p.rows_per_wg;
        if (r0 + p.rows_per_wg <= 0 || r0 >= nrows) return false;
      }
    }
    wrow0 = r0 + 32 * (MODE == kDense ? wave / HW : wave);
    wg_rows_end = min(r0 + p.rows_per_wg, nrows);
    wave_rows = wrow0 < wg_rows_end && wrow0 + 32 > 0;

    past = 0;
    if (MODE == kDense) {
      // (the same value in every lane: made scalar, as the tile bounds are)
      const int len_b = (b < nlens) ? __builtin_amdgcn_readfirstlane(lens[b]) : p.lens[b];
      n_keys = p.causal ? len_b + 1 : p.S;
      if (p.has_past) past = n_keys - p.S;
      rot_past = past;
      if (p.win_cap > 0) {
        // sliding-window cache: keys are the buffer's rows after the eviction,
        // masks work in row coordinates, rotary in absolute positions
        n_keys = window_geom(len_b + 1, p.S, p.win_cap).fill;
        past = n_keys - p.S;
      }
    } else if (MODE == kCsr) {
      n_keys = p.key_total[b];
      if (p.has_past) past = n_keys - p.S;
    } else {
      n_keys = nrows;
    }
    if (MODE != kDense) rot_past = past;
    pmin = past + r0;
    pmax = past + wg_rows_end - 1;
    k_lo = 0;
    k_hi = n_keys;
    if (MODE == kDense && p.causal) {
      k_hi = min(n_keys, pmax + 1);
      if (p.window >= 0) k_lo = max(0, pmin - p.window);
    }
    csr_lo = 0;
    layout = 0;
    tiles_per_block = 1;
    if (MODE == kCsr) {
      layout = h % p.num_layout;
      // the row of the block's first query, clamped into the row pointers
      // (a key total beyond max_blocks * block violates a precondition the
      // host cannot check; the reads stay in bounds)
      const int rb = min(max(pmin / p.block, 0), p.max_blocks - 1);
      csr_lo = max(p.rp[layout * p.rp_stride + rb], 0);
      const int csr_hi = min(p.rp[layout * p.rp_stride + rb + 1], (int)p.cols_stride);
      tiles_per_block = p.block > BN ? p.block / BN : 1;
      n_tiles = max(0, csr_hi - csr_lo) * tiles_per_block;
    } else {
      n_tiles = (k_hi > k_lo) ? (k_hi - k_lo + BN - 1) / BN : 0;
    }
    if (MODE == kVarlen) kv_base = row_base * p.k_j + (int64_t)kvh * p.k_h;
    else kv_base = (int64_t)b * p.k_b + (int64_t)kvh * p.k_h;
    return true;
  }

  // keys [start, start + BN) of tile t, of which [start, lim) may be visible
  __device__ TileRange tile(const FlashParams& p, int t) const {
    TileRange r;
    if (MODE == kCsr) {
      const int e = csr_lo + t / tiles_per_block;
      const int c = min(max(p.cols[layout * p.cols_stride + e], 0), p.max_blocks - 1);
      r.start = c * p.block + (t % tiles_per_block) * BN;
      const int blk_end = (c + 1) * p.block;
      r.lim = min(min(r.start + BN, blk_end), min(n_keys, pmax + 1));
    } else {
      r.start = k_lo + t * BN;
      r.lim = min(r.start + BN, k_hi);
    }
    return r;
  }

  // a tile visible to every row of the workgroup needs no mask
  __device__ bool full(const FlashParams& p, const TileRange& r) const {
    bool f = r.lim == r.start + BN;
    if (MODE == kDense && p.causal)
      f = f && r.start + BN - 1 <= pmin && (p.window < 0 || r.start >= pmax - p.window);
    else if (MODE == kCsr)
      f = f && r.start + BN - 1 <= pmin;
    return f;
  }
};

// Waves per SIMD the launch bounds ask for (the second launch-bounds value):
// two where LDS lets that many workgroups share a CU.  4-wave groups
// double-buffer their K/V tiles (two groups per CU); smaller groups keep one
// buffer so that four of them fit.
template <int NW, int HP> struct FlashOcc {
  static constexpr int nbuf = NW >= 4 ? 2 : 1;
  static constexpr int waves_per_simd = (HP <= 128 && NW >= 2) ? 2 : 1;
};

template <typename T, int HP, int BN, int MODE, int NW, bool SOFTCAP>
__global__ __launch_bounds__(64 * NW, (FlashOcc<NW, HP>::waves_per_simd)) void flash_kernel(FlashParams p) {
  using Mma = FlashMma<T, HP>;
  constexpr int KS = Mma::KS, VS = Mma::VS, CH = Mma::CH;
  constexpr int TILE = BN * (KS + VS);
  constexpr int CPR = HP / CH;  // 16-byte chunks per row
  constexpr int nthreads = 64 * NW;
  // chunks (K and V) each thread moves per tile; prefetching a whole tile into
  // registers only when that stays small
  constexpr int CPT = (2 * BN * CPR + nthreads - 1) / nthreads;
  constexpr bool kPrefetch = CPT <= 16;
  constexpr int NBUF = FlashOcc<NW, HP>::nbuf;
  __shared__ __attribute__((aligned(16))) T lds[NBUF * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform (so that everything derived from it stays in scalar registers)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = p.H;
  // ---- workgroup -> (sample, kv head, heads, rows, key tiles) ---------------
  FlashWork<MODE, BN> w;
  if (!w.init(p, wave)) return;
  const int b = w.b, h = w.h, nrows = w.nrows, past = w.past, pmin = w.pmin;
  const int wrow0 = w.wrow0, wg_rows_end = w.wg_rows_end, n_tiles = w.n_tiles;
  const bool wave_rows = w.wave_rows;
  const int64_t row_base = w.row_base, kv_base = w.kv_base;
  auto tile_range = [&](int t) -> TileRange { return w.tile(p, t); };
  const T* qg = static_cast<const T*>(p.q);
  const T* kg = static_cast<const T*>(p.kc);
  const T* vg = static_cast<const T*>(p.vc);

  // ---- queries of this wave (registers) ---------------------------------------
  Mma mma;
  mma.init();
  const int qrow = wrow0 + (lane & 31);
  const bool row_ok = wave_rows && qrow >= 0 && qrow < wg_rows_end;
  // The scores come out of the MFMA already as the softmax exponent
  // (log2 domain): the query carries scale * log2(e), or, with a softcap c,
  // 2 * log2(e) * scale / c, the argument of the exp2 inside tanh.
  const float cap = p.softcap;
  // the softcap instance is launched only with a positive cap
  constexpr bool use_cap = SOFTCAP;
  // float32 storage evaluates tanh to float32 accuracy near zero (the float16
  // path keeps the shorter formula: its probabilities are rounded to f16)
  constexpr bool kExactCap = std::is_same<T, float>::value;
  const float qscale = use_cap ? 2.f * kLog2e * p.scale / cap : kLog2e * p.scale;
  const float capA = cap * kLog2e, capB = 2.f * cap * kLog2e;
  {
    const int rr = min(max(qrow, 0), nrows - 1);
    const T* qp = (MODE == kVarlen)
                      ? qg + (row_base + rr) * p.q_s + (int64_t)h * p.q_h
                      : qg + (int64_t)b * p.q_b + (int64_t)rr * p.q_s + (int64_t)h * p.q_h;
    prep_query(mma, qp, w.rot_past + rr, p, qscale, lane);
  }
  const int pos = past + qrow;  // absolute position of this lane's query

  // ---- tile loader: 16-byte chunks (K rows then V rows) -> LDS ----------------
  auto chunk_src = [&](const TileRange& r, int idx, bool& zero) -> const T* {
    const bool isv = idx >= BN * CPR;
    const int ci = isv ? idx - BN * CPR : idx;
    const int row = ci / CPR, d = (ci % CPR) * CH;
    const int last = min(max(r.start, r.lim - 1), p.kv_rows - 1);
    const int grow = min(r.start + row, last);
    zero = d >= H;
    return (isv ? vg : kg) + kv_base + (int64_t)grow * p.k_j + d;
  };
  auto chunk_dst = [&](int buf, int idx) -> T* {
    T* base = lds + buf * TILE;
    const bool isv = idx >= BN * CPR;
    const int ci = isv ? idx - BN * CPR : idx;
    const int row = ci / CPR, d = (ci % CPR) * CH;
    return isv ? base + BN * KS + row * VS + d : base + row * KS + d;
  };
  // Prefetch path: thread tid moves chunks tid + u * nthreads, u < CPT; the
  // first KU are K chunks, the rest V chunks, all at column d0 of rows
  // row0 + RSTEP * (u % KU), so per tile only the first row moves.
  constexpr int KU = (BN * CPR) / nthreads;   // K chunks per thread
  constexpr int RSTEP = nthreads / CPR;
  static_assert(!kPrefetch || (BN * CPR) % nthreads == 0, "whole K/V chunk rows per thread");
  const int row0 = tid / CPR, d0 = (tid % CPR) * CH;
  const bool zero_col = d0 >= H;  // columns beyond the head stay zero in LDS
  const bool pad_cols = H < HP;   // uniform: only then can zero_col be true
  // Every lane loads (a column past the head reads column 0 instead), so all
  // paths issue the same loads; those lanes skip the store, and the columns
  // past the head stay as zeroed here.
  const int dload = zero_col ? 0 : d0;
  if (kPrefetch && pad_cols) {
    for (int i = tid; i < NBUF * TILE * (int)sizeof(T) / 16; i += nthreads)
      reinterpret_cast<uint4v*>(lds)[i] = uint4v{0u, 0u, 0u, 0u};
    __syncthreads();
  }
  const int kj = (int)p.k_j;      // row stride (elements); a slab of rows fits 32 bits
  uint4v stage[kPrefetch ? CPT : 1];
  // Prefetch depth: with short per-tile compute (64-dim heads) the next
  // tile's loads would not return in time, so those kernels load two tiles
  // ahead into a second register stage.
  constexpr int kStages = (kPrefetch && HP <= 64) ? 2 : 1;
  uint4v stage2[kStages == 2 ? CPT : 1];
  // Quantised caches (float32 dense prompts): the tiles are read as codes (4 bytes
  // of int8 or 2 bytes of nibbles per 4-element chunk) and widened to
  // code * scale, the product the prep of a float cache would store, as they
  // go into LDS.  A thread's columns are fixed, so are its scales.
  constexpr bool kQ = std::is_same<T, float>::value && MODE == kDense && kPrefetch;
  const int qb = kQ ? p.qbits : 0;
  float ksc[4] = {0.f, 0.f, 0.f, 0.f}, vsc[4] = {0.f, 0.f, 0.f, 0.f};
  if (kQ && qb != 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = min(dload + i, H - 1);
      ksc[i] = p.qk_pc ? p.qk_scale[(int64_t)w.kvh * H + d] : p.qk_scale[0];
      vsc[i] = p.qv_pc ? p.qv_scale[(int64_t)w.kvh * H + d] : p.qv_scale[0];
    }
  }
  auto widen = [&](uint32_t word, const float (&sc)[4]) -> uint4v {
    float f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = qb == 8 ? (int)(int8_t)(word >> (8 * i)) : (int)((word >> (4 * i)) & 15u) - 8;
      f[i] = (float)c * sc[i];
    }
    return uint4v{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
  };
  auto load_tile_to = [&](int t, uint4v* dst) {
    const TileRange r = tile_range(t);
    // uniform base at the tile's first row; per-thread 32-bit offsets
    const int last = min(max(r.start, r.lim - 1), p.kv_rows - 1) - r.start;
    if (kQ && qb != 0) {
      // element e of the code caches sits at byte e (int8) or e / 2 (int4)
      const int sh = qb == 4 ? 1 : 0;
      const int64_t e0 = kv_base + (int64_t)r.start * p.k_j;
      const uint8_t* kt8 = static_cast<const uint8_t*>(p.kc) + (e0 >> sh);
      const uint8_t* vt8 = static_cast<const uint8_t*>(p.vc) + (e0 >> sh);
#pragma unroll
      for (int u = 0; u < (kPrefetch ? CPT : 1); ++u) {
        const int off = (min(row0 + RSTEP * (u % KU), last) * kj + dload) >> sh;
        const uint8_t* src = (u < KU ? kt8 : vt8) + off;
        const uint32_t word = qb == 8 ? *reinterpret_cast<const uint32_t*>(src)
                                      : (uint32_t)*reinterpret_cast<const uint16_t*>(src);
        dst[u] = uint4v{word, 0u, 0u, 0u};
      }
      return;
    }
    const T* kt = kg + kv_base + (int64_t)r.start * p.k_j;
    const T* vt = vg + kv_base + (int64_t)r.start * p.k_j;
#pragma unroll
    for (int u = 0; u < (kPrefetch ? CPT : 1); ++u) {
      const int off = min(row0 + RSTEP * (u % KU), last) * kj + dload;
      const T* src = (u < KU ? kt : vt) + off;
      dst[u] = *reinterpret_cast<const uint4v*>(src);
    }
  };
  auto load_tile = [&](int t) { load_tile_to(t, stage); };
  auto store_tile_from = [&](int buf, const uint4v* srcs) {
    T* base = lds + buf * TILE;
#pragma unroll
    for (int u = 0; u < (kPrefetch ? CPT : 1); ++u) {
      const int row = row0 + RSTEP * (u % KU);
      T* dst = u < KU ? base + row * KS + d0 : base + BN * KS + row * VS + d0;
      if (!(pad_cols && zero_col))
        *reinterpret_cast<uint4v*>(dst) = (kQ && qb != 0) ? widen(srcs[u][0], u < KU ? ksc : vsc) : srcs[u];
    }
  };
  auto store_tile = [&](int buf) { store_tile_from(buf, stage); };
  // direct copy without holding a whole tile in registers (large tiles per thread)
  auto copy_tile = [&](int t, int buf) {
    const TileRange r = tile_range(t);
    for (int idx = tid; idx < 2 * BN * CPR; idx += nthreads) {
      bool zero;
      const T* src = chunk_src(r, idx, zero);
      uint4v v = zero ? uint4v{0u, 0u, 0u, 0u} : *reinterpret_cast<const uint4v*>(src);
      *reinterpret_cast<uint4v*>(chunk_dst(buf, idx)) = v;
    }
  };

  const T* bias = static_cast<const T*>(p.bias);
  int64_t bias_row = 0;
  int pad_q = 0;
  if (bias != nullptr) {
    if (MODE == kVarlen) {
      pad_q = p.token_offset[row_base + min(qrow, nrows - 1)] - b * p.pad_seq;
      pad_q = min(max(pad_q, 0), p.pad_seq - 1);
      bias_row = (int64_t)b * p.bias_sb + (int64_t)h * p.bias_sh + (int64_t)pad_q * p.bias_ss;
    } else {
      bias_row = (int64_t)b * p.bias_sb + (int64_t)h * p.bias_sh + (int64_t)min(qrow, nrows - 1) * p.bias_ss;
    }
  }

  float m = kNegInf, lsum = 0.f;
  if (kPrefetch && n_tiles > 0) {
    load_tile(0);
    store_tile(0);
    if (kStages == 2) load_tile(min(1, n_tiles - 1));  // stage: tile 1
    __syncthreads();
  }
  // Scores, online softmax and PV of one tile whose K and V rows sit in LDS.
  auto compute = [&](const TileRange& r, const T* Kt, const T* Vt) {
    const bool plain = w.full(p, r) && bias == nullptr;  // uniform: no per-score mask or bias
    float16v sacc[BN / 32];
    if constexpr (std::is_same<T, f16>::value && BN == 64) {
      mma.qk_tile64(Kt, lane, sacc);
    } else {
#pragma unroll
      for (int blk = 0; blk < BN / 32; ++blk) sacc[blk] = mma.qk_block(Kt, 32 * blk, lane);
    }
    mfma_result_fence();
    // softcap: c * log2(e) * tanh(y) = A - B / (2^u + 1) with u = 2 * log2(e) * y.
    // A plain tile keeps its raw scores: the cap is monotone, so the capped
    // maximum is the cap of the raw one, and the cap is applied in the exponent.
    if (!plain && bias == nullptr) {
      // score (blk, i) of this lane is key kb + c, c = 32 blk + 8 (i / 4) + i % 4
      // a constant, so the masks reduce to a range [clo, chi] of c per lane
      const int kb = r.start + 4 * (lane >> 5);
      int clo = 0, chi = r.lim - 1 - kb;
      if ((MODE == kDense && p.causal) || MODE == kCsr) chi = min(chi, pos - kb);
      if (MODE == kDense && p.causal && p.window >= 0) clo = pos - p.window - kb;
      if (!row_ok) chi = -1;
#pragma unroll
      for (int blk = 0; blk < BN / 32; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = 32 * blk + 8 * (i >> 2) + (i & 3);
          float v = sacc[blk][i];
          if (use_cap) v = kExactCap ? capA * tanh_from_u(v) : capA - capB * fast_rcp(fast_exp2(v) + 1.f);
          sacc[blk][i] = (c >= clo && c <= chi) ? v : kNegInf;
        }
    } else if (!plain) {
#pragma unroll
      for (int blk = 0; blk < BN / 32; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = r.start + 32 * blk + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          bool ok = row_ok && key < r.lim;
          if (MODE == kDense) {
            if (p.causal) {
              ok = ok && key <= pos;
              if (p.window >= 0) ok = ok && key >= pos - p.window;
            }
          } else if (MODE == kCsr) {
            ok = ok && key <= pos;
          }
          float v = sacc[blk][i];
          if (use_cap) v = kExactCap ? capA * tanh_from_u(v) : capA - capB * fast_rcp(fast_exp2(v) + 1.f);
          if (bias != nullptr && ok) {
            if (MODE == kVarlen) {
              int pad_k = p.token_offset[row_base + key] - b * p.pad_seq;
              pad_k = min(max(pad_k, 0), p.pad_seq - 1);
              v += kLog2e * to_f32(bias[bias_row + pad_k]);
            } else if (key < p.bias_cols) {
              v += kLog2e * to_f32(bias[bias_row + key]);
            }
          }
          sacc[blk][i] = ok ? v : kNegInf;
        }
    }
    float tmax = kNegInf;
#pragma unroll
    for (int blk = 0; blk < BN / 32; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[blk][i]);
    if (use_cap && plain)
      tmax = kExactCap ? capA * tanh_from_u(tmax) : capA - capB * fast_rcp(fast_exp2(tmax) + 1.f);
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    // The running max m moves only when a score exceeds it by more than
    // kMaxSlack (log2 units): probabilities then stay <= 2^kMaxSlack, exact
    // enough in fp16 and far from overflow, and O is rescaled rarely.
    const bool grow = tmax > m + kMaxSlack;
    if (__any(grow)) {
      // a side effect keeps this a branch: executed unconditionally, the
      // rescale of O would cost a multiply per accumulator on every tile
      asm volatile("" ::: "memory");
      const float mnew = grow ? tmax : m;
      const float alpha = (mnew == kNegInf) ? 1.f : fast_exp2(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < Mma::ND; ++db) mma.o[db] *= alpha;
    }
    const float muse = (m == kNegInf) ? 0.f : m;
    // probabilities: on a plain softcap tile the cap and the max subtraction
    // share one FMA; otherwise the scores already hold the exponent
    const float c0 = capA - muse;
    if constexpr (std::is_same<T, f16>::value && BN == 64) {
      // P in f16 (the PV operand); the row sum adds the same rounded values
      half8v pb[4];
      if (use_cap && plain) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < 8; ++i)
            pb[q][i] = (f16)fast_exp2(c0 - capB * fast_rcp(fast_exp2(sacc[q >> 1][8 * (q & 1) + i]) + 1.f));
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < 8; ++i) pb[q][i] = (f16)fast_exp2(sacc[q >> 1][8 * (q & 1) + i] - muse);
      }
      const half2v one2 = {(f16)1.f, (f16)1.f};
      float ps[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ps[q] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          ps[q] = __builtin_amdgcn_fdot2(half2v{pb[q][2 * j], pb[q][2 * j + 1]}, one2, ps[q], false);
      }
      lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);
      mma.pv_tile64(Vt, pb, lane);
    } else {
      float pr[BN / 32][16];
      if (use_cap && plain) {
#pragma unroll
        for (int blk = 0; blk < BN / 32; ++blk)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            pr[blk][i] = kExactCap ? fast_exp2(capA * tanh_from_u(sacc[blk][i]) - muse)
                                   : fast_exp2(c0 - capB * fast_rcp(fast_exp2(sacc[blk][i]) + 1.f));
      } else {
#pragma unroll
        for (int blk = 0; blk < BN / 32; ++blk)
#pragma unroll
          for (int i = 0; i < 16; ++i) pr[blk][i] = fast_exp2(sacc[blk][i] - muse);
      }
      float psum = 0.f;
#pragma unroll
      for (int blk = 0; blk < BN / 32; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) psum += pr[blk][i];
      lsum += psum;
#pragma unroll
      for (int blk = 0; blk < BN / 32; ++blk) mma.pv_block(Vt, 32 * blk, pr[blk], lane);
    }
  };
  // One tile: compute tile t from LDS; `cur` holds tile t + 1 (two-stage
  // prefetch) and `nxt` receives tile t + 2.  Loads past the last tile re-read
  // it, so every path issues the same loads.
  auto tile_step = [&](int t, uint4v* cur, uint4v* nxt) {
    const int buf = NBUF == 2 ? (t & 1) : 0;
    load_tile_to(min(t + 2, n_tiles - 1), nxt);
    compute(tile_range(t), lds + buf * TILE, lds + buf * TILE + BN * KS);
    if (t + 1 < n_tiles) {
      if (NBUF == 1) __syncthreads();  // every wave is done with the one buffer
      store_tile_from(NBUF == 2 ? buf ^ 1 : 0, cur);
    }
    __syncthreads();
  };
  if constexpr (kStages == 2) {
    for (int t = 0; t < n_tiles; t += 2) {
      tile_step(t, stage, stage2);
      if (t + 1 < n_tiles) tile_step(t + 1, stage2, stage);
    }
  } else {
    for (int t = 0; t < n_tiles; ++t) {
      const int buf = NBUF == 2 ? (t & 1) : 0;
      if (kPrefetch) {
        if (t + 1 < n_tiles) load_tile(t + 1);
      } else {
        // with two buffers, buf was last read two tiles ago and every wave has
        // passed the barrier that followed that tile; with one, wait for the
        // readers of the previous tile
        if (NBUF == 1 && t > 0) __syncthreads();
        copy_tile(t, buf);
        __syncthreads();
      }
      compute(tile_range(t), lds + buf * TILE, lds + buf * TILE + BN * KS);
      if (kPrefetch) {
        if (t + 1 < n_tiles) {
          if (NBUF == 1) __syncthreads();  // every wave is done with the one buffer
          store_tile(NBUF == 2 ? buf ^ 1 : 0);
        }
        __syncthreads();
      }
    }
  }

  // ---- normalise and store -----------------------------------------------------
  mfma_result_fence();
  if (!wave_rows) return;
  lsum += shfl_xor(lsum, 32);
  bool has_sink = false;
  float sg = 0.f;
  if (p.sink != nullptr) {
    has_sink = true;
    sg = kLog2e * to_f32(static_cast<const T*>(p.sink)[h]);
  } else if (p.smooth == 1) {
    has_sink = true;
  }
  float inv;
  if (lsum == 0.f) {
    inv = 0.f;
  } else if (has_sink) {
    const float M2 = fmaxf(m, sg);
    const float den = lsum * fast_exp2(m - M2) + fast_exp2(sg - M2);
    inv = fast_exp2(m - M2) / den;
  } else {
    inv = 1.f / lsum;
  }
  if (!row_ok) return;
  T* og = static_cast<T*>(p.out);
  T* orow = (MODE == kVarlen) ? og + (row_base + qrow) * p.o_s + (int64_t)h * p.o_h
                              : og + (int64_t)b * p.o_b + (int64_t)qrow * p.o_s + (int64_t)h * p.o_h;
#pragma unroll
  for (int db = 0; db < Mma::ND; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = 32 * db + 8 * gq + 4 * (lane >> 5);
      if (d < H) {
#pragma unroll
        for (int i = 0; i < 4; ++i) orow[d + i] = from_f32<T>(mma.o[db][4 * gq + i] * inv);
      }
    }
}

// ---------------------------------------------------------------------------
// LDS tiles of the ping-pong f16 kernel (64-key tiles, heads of 64 or 128).
//
// K and V tiles go straight from global memory into LDS (global_load_lds, 16
// bytes per lane; no register staging), two buffers each.
//
// LDS rows: K rows are padded by one 16-byte chunk (the score operand reads
// of 16 consecutive rows then hit distinct banks); V rows are unpadded with
// their 16-byte chunks XOR-swizzled by row, which keeps the transposing PV
// operand reads conflict-free.  A global_load_lds instruction fills 64
// consecutive 16-byte slots, so every slot, padding included, is loaded (a
// padding slot repeats chunk 0 of its row).
template <int HP> struct PipeLayout {
  static constexpr int BN = 64;
  static constexpr int CPR = HP / 8;              // 16-byte chunks per row
  static constexpr int KS = HP + 8;               // K row stride (elements)
  static constexpr int KTILE = BN * KS;           // elements
  static constexpr int VTILE = BN * HP;
  static constexpr int NKI = KTILE * 2 / 1024;    // 1 KiB wave loads per K tile (CPR + 1)
  static constexpr int NVI = VTILE * 2 / 1024;    // per V tile (CPR)
  // chunk swizzle of V row r: the rows one transposing read touches (four
  // consecutive rows, and rows 8 apart) differ in it or in their bank half
  __device__ static constexpr int swv_of_ir(int ir) { return HP >= 128 ? ir : ((ir >> 1) & 1); }
  __device__ static int swv(int r) { return 4 * swv_of_ir(r & 3); }
};

// Calls f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>).
template <typename F, int... Is>
__device__ __forceinline__ void pipe_static_for(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}

// Transposing LDS read of 4 f16 (ds_read_b64_tr_b16) at byte address
// addr + OFF, issued as a volatile statement with its wait made explicit
// (lds_wait_tr): the compiler's own wait counting treats the transposing
// builtin as an access of unknown memory and makes it wait for every
// outstanding global-to-LDS copy, which would stall each PV phase behind the
// copies of the next tiles.  LDS operations complete in issue order, so a wait
// until at most n LDS operations are outstanding covers every read issued
// before the last n (a scalar load in between only makes the wait longer).
// Volatile statements keep their order, and the wait takes the read results as
// operands, so nothing reads them before it.
template <int OFF>
__device__ __forceinline__ uint2v lds_tr16_asm(uint32_t addr) {
  uint2v r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void lds_wait_tr(uint2v& a, uint2v& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}

// Global-to-LDS copy of 16 bytes per lane (global_load_lds_dwordx4) from
// byte address base + off (base uniform, in SGPRs; off per lane): lane l's
// bytes land at LDS byte address lds + 16 l.  Issued as a volatile statement:
// with a copy into LDS outstanding, the compiler's wait counting would wait
// for all LDS reads at once instead of by count.  The copies are waited for
// explicitly (vmcnt(0) before the barrier that publishes each tile).
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}

// ds_read_b128 at byte address addr + OFF, issued as a volatile statement
// whose wait is explicit (lds_wait_b128), as for the transposing reads.
template <int OFF>
__device__ __forceinline__ uint4v lds_b128_asm(uint32_t addr) {
  uint4v r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void lds_wait_b128(uint4v& a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "i"(N));
}

// The MFMA phase of the ping-pong kernel: the PV MFMAs of one tile
// (probabilities pb, V buffer VB) and the score MFMAs of the next (K buffer
// KB), interleaved one to one, with the LDS operand reads of D pairs of MFMAs
// in flight, and the phase's NDMA global-to-LDS copies (dma(i)) spread over
// the pairs, so that the copies queue behind MFMAs rather than ahead of them.  Pair j is score MFMA j (k-step j / 2, key block j % 2) and PV
// MFMA j (16-key group j / ND, output block j % ND).  LDS reads complete in
// issue order, so the wait before each MFMA counts the reads issued after its
// own operands.  kaddr: this lane's byte address of its first score operand
// in K buffer 0; vaddr[db]: its byte address of output block db's PV
// operand in V buffer 0.
template <int HP, int VB, int KB, bool DO_PV, bool DO_QK, int D, int NDMA, typename DMA>
__device__ __forceinline__ void mphase(float16v (&o)[HP / 32], float16v (&sc)[2],
                                       const uint32_t (&vaddr)[HP / 32], uint32_t kaddr,
                                       const half8v (&pb)[4], const half8v (&qf)[HP / 16], DMA&& dma) {
  using L = PipeLayout<HP>;
  constexpr int ND = HP / 32, NS = HP / 16;
  constexpr int N = 4 * ND;
  static_assert(N == 2 * NS, "as many score as PV MFMAs per tile");
  constexpr int VOFF = VB * L::VTILE * 2, KOFF = KB * L::KTILE * 2;
  constexpr int RQ = DO_QK ? 1 : 0, RP = DO_PV ? 2 : 0, RJ = RQ + RP;  // reads per pair
  uint4v kr[N];
  uint2v lo[N], hi[N];
  if (DO_QK) {
    sc[0] = float16v{};
    sc[1] = float16v{};
  }
  auto issue = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if constexpr (DO_QK) kr[j] = lds_b128_asm<KOFF + (j % 2) * 64 * L::KS + 32 * (j / 2)>(kaddr);
    if constexpr (DO_PV) {
      constexpr int q = j / ND, db = j % ND;
      lo[j] = lds_tr16_asm<VOFF + 32 * q * HP>(vaddr[db]);
      hi[j] = lds_tr16_asm<VOFF + 32 * q * HP + 16 * HP>(vaddr[db]);
    }
  };
  auto issue_q = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    kr[j] = lds_b128_asm<KOFF + (j % 2) * 64 * L::KS + 32 * (j / 2)>(kaddr);
  };
  auto issue_p = [&](auto jc) {
    constexpr int j = decltype(jc)::value, q = j / ND, db = j % ND;
    lo[j] = lds_tr16_asm<VOFF + 32 * q * HP>(vaddr[db]);
    hi[j] = lds_tr16_asm<VOFF + 32 * q * HP + 16 * HP>(vaddr[db]);
  };
  pipe_static_for(issue, std::make_integer_sequence<int, (D < N ? D : N)>{});
  pipe_static_for(
      [&](auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int last = (j + D - 1 < N - 1) ? j + D - 1 : N - 1;  // last pair issued in full
        constexpr bool more = j + D < N;
        if constexpr (DO_QK) {
          lds_wait_b128<RP + RJ * (last - j)>(kr[j]);
          sc[j % 2] = mfma32x32x16(__builtin_bit_cast(half8v, kr[j]), qf[j / 2], sc[j % 2]);
          if constexpr (more) issue_q(std::integral_constant<int, j + D>{});
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (DO_PV) {
          constexpr int q = j / ND, db = j % ND;
          lds_wait_tr<RJ * (last - j) + ((DO_QK && more) ? 1 : 0)>(lo[j], hi[j]);
          const uint4v u = {lo[j][0], lo[j][1], hi[j][0], hi[j][1]};
          o[db] = mfma32x32x16(__builtin_bit_cast(half8v, u), pb[q], o[db]);
          if constexpr (more) issue_p(std::integral_constant<int, j + D>{});
          __builtin_amdgcn_sched_barrier(0);
        }
        // copies i with i * N / NDMA == j go out after pair j
        pipe_static_for(
            [&](auto ic) {
              constexpr int i = decltype(ic)::value;
              if constexpr (i * N / NDMA == j) dma(ic);
            },
            std::make_integer_sequence<int, NDMA>{});
        __builtin_amdgcn_sched_barrier(0);
      },
      std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------------------
// Ping-pong f16 kernel (64-key tiles, heads of 64 or 128): two work items per
// workgroup of eight waves, one per group of four waves (waves 0-3 and 4-7,
// so that wave j of one group shares a SIMD with wave j of the other).  Each
// group streams its own K/V tiles (global-to-LDS copies, two buffers each,
// the layout above) and runs its item in two kinds of phase separated by
// workgroup barriers:
//   M(s): the PV MFMAs of tile s - 1 and the score MFMAs of tile s (and the
//         copies of K(s + 1) and V(s) into LDS);
//   V(s): the softmax of tile s: masks, softcap, running maximum, exp2, row
//         sums (vector ALU only).
// The second group runs one phase behind the first, so on every SIMD one wave
// issues MFMAs while the other keeps the vector ALU busy.  A group with fewer
// tiles idles through the remaining phases; every wave passes every barrier.
template <int HP, int MODE, bool SOFTCAP>
__global__ __launch_bounds__(512, 1) void flash_pp_kernel(FlashParams p, int gx, int gy, int gz) {
  using Mma = FlashMma<f16, HP>;
  using L = PipeLayout<HP>;
  constexpr int NW = 4;   // waves per group
  constexpr int BN = 64;
  static_assert(L::KS == Mma::KS, "score operand reads use the padded K rows");
  constexpr int MK = (L::NKI + NW - 1) / NW;   // K copies per wave per tile
  constexpr int MV = (L::NVI + NW - 1) / NW;   // V copies per wave per tile
  constexpr int GL = 2 * L::KTILE + 2 * L::VTILE;   // elements of one group's tiles
  __shared__ __attribute__((aligned(1024))) f16 lds[2 * GL];
  static_assert(2 * (L::VTILE + 3 * 16 * HP + 8 * HP) < 65536, "V read offsets fit the immediate");

  const int n_items = gx * gy * gz;
  const int NPH = (gy + 1) / 2;
  static_assert(MODE == kDense, "the ping-pong kernel serves dense prompts");
  const int npairs = gx * NPH * gz;
  const int G = gridDim.x, wg = blockIdx.x;
  const int wx = (G % 8 == 0) ? (wg % 8) * (G / 8) + wg / 8 : wg;
  const int S = NPH * gz;  // dense: slab pairs
  const bool xcd_slabs = S % 8 == 0 && G % 8 == 0;
  // the samples' lengths (dense), read once per workgroup: every round needs
  // them again, and a global load there would cost a memory latency
  constexpr int kLensMax = 1024;
  __shared__ int s_lens[kLensMax];
  const int nlens = min(p.B, kLensMax);
  for (int i = threadIdx.x; i < nlens; i += 512) s_lens[i] = p.lens[i];
  __syncthreads();
  // The output of a round waits in LDS (each wave's 32 x HP tile, row-major,
  // 16-byte chunks XOR-swizzled by row, in its quarter of the group's V
  // buffers) and is stored once the next round's query loads are out, in
  // whole-row 16-byte chunks: the stores' latency then overlaps theirs.
  constexpr int OCH = HP / 8, OSW = OCH < 16 ? OCH - 1 : 15;  // chunks per row, swizzle mask
  static_assert(4 * 32 * HP <= 2 * L::VTILE, "the group's outputs fit its V buffers");
  // per wave: rows pending (0: none) and the output address of the first
  // one, kept in LDS rather than in registers through the tile loop
  __shared__ int s_pend_rows[8];
  __shared__ f16* s_pend_base[8];
  if ((threadIdx.x & 63) == 0) s_pend_rows[threadIdx.x >> 6] = 0;  // wave-private
  auto store_pending = [&](const f16* stage) {
    const int wv8 = threadIdx.x >> 6;
    int ln = threadIdx.x & 63;
    asm volatile("" : "+v"(ln));  // per-lane addresses are made here, not held across rounds
    const int rows = __builtin_amdgcn_readfirstlane(s_pend_rows[wv8]);
    if (rows > 0) {
      f16* base = s_pend_base[wv8];
#pragma unroll
      for (int k = 0; k < 32 * OCH / 64; ++k) {
        const int c = ln + 64 * k, r = c / OCH, cc = c - r * OCH;
        const half8v v = *reinterpret_cast<const half8v*>(stage + r * HP + 8 * (cc ^ (r & OSW)));
        if (r < rows && 8 * cc < p.H) *reinterpret_cast<half8v*>(base + r * p.o_s + 8 * cc) = v;
      }
      if (ln == 0) s_pend_rows[wv8] = 0;
    }
  };
  for (int round = 0;; ++round) {
  // per-lane values are recomputed in every round rather than held across
  // the loop (register pressure)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wv >> 2;   // group
  const int wave = wv & 3;   // wave within the group
  const int H = p.H;
  auto lds_byte = [](const f16* q) {
    return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const f16*)q);
  };
  f16* const K0 = lds + grp * GL;
  f16* const K1 = K0 + L::KTILE;
  f16* const V0 = K0 + 2 * L::KTILE;
  f16* const V1 = V0 + L::VTILE;

  // ---- the workgroup's pairs of items ------------------------------------------
  // At most one workgroup per CU, looping over pairs of items, mirrored on odd
  // rounds so that the long pairs of one round meet the short pairs of the
  // next.  Pairs = (row block, slab pair), a slab pair being a sample and a pair of adjacent head groups, row blocks taken latest
  // first (the most keys under a causal bound).  When the slab pairs split evenly over the
  // eight XCDs, each XCD takes its own slab pairs through all row blocks: the
  // rows in flight on one XCD then share the K/V windows of a few slabs, which
  // stay in its L2.  Otherwise round k gives workgroup w the pair k G + w', w'
  // its rank in an XCD-contiguous order.
  int f = round * G + ((round & 1) ? G - 1 - wx : wx);
  int rbi = 0, sp = 0;
  if (xcd_slabs) {
    const int NB = S / 8, G8 = G / 8, wl = wg / 8;
    const int q = round * G8 + ((round & 1) ? G8 - 1 - wl : wl);
    if (q >= gx * NB) break;
    rbi = q / NB;
    sp = (wg % 8) * NB + (q - rbi * NB);
  } else {
    if (f >= npairs) break;
    rbi = f / S;
    sp = f - rbi * S;
  }
  int id_own, id_other;
  {
    const int bb = sp / NPH, jp = sp - bb * NPH;
    const int base = rbi + gx * gy * bb;
    id_own = (2 * jp + grp < gy) ? base + gx * (2 * jp + grp) : n_items;
    id_other = (2 * jp + (grp ^ 1) < gy) ? base + gx * (2 * jp + (grp ^ 1)) : n_items;
  }
  FlashWork<MODE, BN> w{}, wo{};
  const bool live = w.init_item(p, wave, id_own, gx, gy, gz, s_lens, nlens);
  const bool live_o = wo.init_item(p, wave, id_other, gx, gy, gz, s_lens, nlens);
  const int n_tiles = live ? w.n_tiles : 0;
  const int n_steps = max(n_tiles, live_o ? wo.n_tiles : 0);   // the same in every wave
  const int b = w.b, h = w.h, nrows = w.nrows, past = w.past;
  const f16* kg = static_cast<const f16*>(p.kc) + (live ? w.kv_base : 0);
  const f16* vg = static_cast<const f16*>(p.vc) + (live ? w.kv_base : 0);
  const int kj = (int)p.k_j;

  // ---- per-lane copy slots ---------------------------------------------------
  auto k_slot = [&](int u, int& r, int& col) {
    const int j = 64 * (wave + NW * u) + lane;
    r = j / (L::CPR + 1);
    const int pc = j - r * (L::CPR + 1);
    int cc = pc < L::CPR ? pc : 0;
    if (8 * cc >= H) cc = 0;
    col = 8 * cc;
  };
  auto v_slot = [&](int u, int& r, int& col) {
    const int j = 64 * (wave + NW * u) + lane;
    r = j / L::CPR;
    int cc = (j % L::CPR) ^ L::swv(r);
    if (8 * cc >= H) cc = 0;
    col = 8 * cc;
  };
  int koff[MK], voff[MV];
#pragma unroll
  for (int u = 0; u < MK; ++u) {
    int r, col;
    k_slot(u, r, col);
    koff[u] = r * kj + col;
  }
#pragma unroll
  for (int u = 0; u < MV; ++u) {
    int r, col;
    v_slot(u, r, col);
    voff[u] = r * kj + col;
  }
  // a tile with fewer valid rows repeats its last valid row
  auto load_k = [&](int t, f16* dst) {
    const TileRange r = w.tile(p, t);
    const int last = min(max(r.start, r.lim - 1), p.kv_rows - 1) - r.start;
    const f16* src = kg + (int64_t)r.start * p.k_j;
    const bool whole = last == BN - 1;
#pragma unroll
    for (int u = 0; u < MK; ++u) {
      if (wave + NW * u < L::NKI) {
        int off = koff[u];
        if (!whole) {
          int rr, col;
          k_slot(u, rr, col);
          off = min(rr, last) * kj + col;
        }
        lds_dma16(src, 2u * (uint32_t)off, lds_byte(dst + 512 * (wave + NW * u)));
      }
    }
  };
  auto load_v = [&](int t, f16* dst) {
    const TileRange r = w.tile(p, t);
    const int last = min(max(r.start, r.lim - 1), p.kv_rows - 1) - r.start;
    const f16* src = vg + (int64_t)r.start * p.k_j;
    const bool whole = last == BN - 1;
#pragma unroll
    for (int u = 0; u < MV; ++u) {
      if (wave + NW * u < L::NVI) {
        int off = voff[u];
        if (!whole) {
          int rr, col;
          v_slot(u, rr, col);
          off = min(rr, last) * kj + col;
        }
        lds_dma16(src, 2u * (uint32_t)off, lds_byte(dst + 512 * (wave + NW * u)));
      }
    }
  };
  // byte addresses of this lane's PV operand reads in V0, per output block
  uint32_t vaddr[Mma::ND];
  {
    const int G = lane >> 4, t = lane & 15, cc = t & 3, ir = t >> 2;
    const int wsw = L::swv_of_ir(ir);
    const uint32_t v0 = lds_byte(V0);
#pragma unroll
    for (int db = 0; db < Mma::ND; ++db)
      vaddr[db] = v0 + 2u * (uint32_t)((4 * (G >> 1) + ir) * HP + 16 * (G & 1) + 4 * cc + 32 * (db ^ wsw));
  }

  // ---- queries of this wave --------------------------------------------------
  Mma mma;
  const int qrow = w.wrow0 + (lane & 31);
  const bool row_ok = live && w.wave_rows && qrow < w.wg_rows_end;
  const float cap = p.softcap;
  constexpr bool use_cap = SOFTCAP;  // launched only with a positive cap
  const float qscale = use_cap ? 2.f * kLog2e * p.scale / cap : kLog2e * p.scale;
  const float capA = cap * kLog2e, capB = 2.f * cap * kLog2e;
  {
    const int rr = min(qrow, nrows - 1);
    const f16* qg = static_cast<const f16*>(p.q);
    const f16* qp = qg + (int64_t)b * p.q_b + (int64_t)rr * p.q_s + (int64_t)h * p.q_h;
    // the previous round's stores and this round's query loads are in flight
    // together (one wait covers both)
    store_pending(V0 + wave * 32 * HP);
    if (live) prep_query(mma, qp, w.rot_past + rr, p, qscale, lane);
  }
  mma.init();
  const int pos = past + qrow;
  const f16* bias = static_cast<const f16*>(p.bias);
  int64_t bias_row = 0;
  if (bias != nullptr && live)
    bias_row = (int64_t)b * p.bias_sb + (int64_t)h * p.bias_sh + (int64_t)min(qrow, nrows - 1) * p.bias_ss;

  // ---- softmax of one tile (vector ALU) -----------------------------------------
  auto mask_scores = [&](const TileRange& r, float16v (&sc)[2]) {
    if (bias == nullptr) {
      // score (blk, i) of this lane is key kb + c, c = 32 blk + 8 (i / 4) + i % 4,
      // a constant, so the masks reduce to a range [clo, chi] of c per lane
      const int kb = r.start + 4 * (lane >> 5);
      int clo = 0, chi = r.lim - 1 - kb;
      if ((MODE == kDense && p.causal) || MODE == kCsr) chi = min(chi, pos - kb);
      if (MODE == kDense && p.causal && p.window >= 0) clo = pos - p.window - kb;
      if (!row_ok) chi = -1;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int cc = 32 * blk + 8 * (i >> 2) + (i & 3);
          float v = sc[blk][i];
          if (use_cap) v = capA - capB * fast_rcp(fast_exp2(v) + 1.f);
          sc[blk][i] = (cc >= clo && cc <= chi) ? v : kNegInf;
        }
      return;
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = r.start + 32 * blk + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        bool ok = row_ok && key < r.lim;
        if (MODE == kDense) {
          if (p.causal) {
            ok = ok && key <= pos;
            if (p.window >= 0) ok = ok && key >= pos - p.window;
          }
        } else if (MODE == kCsr) {
          ok = ok && key <= pos;
        }
        float v = sc[blk][i];
        if (use_cap) v = capA - capB * fast_rcp(fast_exp2(v) + 1.f);
        if (bias != nullptr && ok && key < p.bias_cols) v += kLog2e * to_f32(bias[bias_row + key]);
        sc[blk][i] = ok ? v : kNegInf;
      }
  };
  auto raw_max = [&](const float16v (&sc)[2]) -> float {
    float t = kNegInf;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) t = fmaxf(t, sc[blk][i]);
    return t;
  };
  auto raw_min = [&](const float16v (&sc)[2]) -> float {
    float t = -kNegInf;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i = 0; i < 16; ++i) t = fminf(t, sc[blk][i]);
    return t;
  };
  // Softcap tiles whose scores all satisfy |x / c| <= tau take tanh from its
  // odd series through y^3: the next term, 2 y^5 / 15, then changes the
  // exponent c tanh(x / c) by at most c 2 tau^5 / 15 <= 5e-5 (a tenth of the
  // f16 rounding of the probabilities), for tau = min(1/4, (7.5e-4 / c)^(1/5)).
  // In raw scores u = 2 log2(e) x / c the bound is polyU = 2 log2(e) tau.
  const float polyU = use_cap ? 2.f * kLog2e * fminf(0.25f, fast_exp2(0.2f * __log2f(7.5e-4f / cap))) : 0.f;
  float m = kNegInf, lsum = 0.f;
  float16v sc[2];
  half8v pb[4];
  auto softmax = [&](int t) {
    const TileRange r = w.tile(p, t);
    const bool plain = w.full(p, r) && bias == nullptr;
    float tmax;
    bool poly = false;
    if (plain) {
      tmax = raw_max(sc);
      if (use_cap) {
        // the series (one exp2 per score instead of three) where every raw
        // score of the wave's tile is small
        poly = __all(fmaxf(tmax, -raw_min(sc)) <= polyU);
        tmax = capA - capB * fast_rcp(fast_exp2(tmax) + 1.f);
      }
    } else {
      mask_scores(r, sc);
      tmax = raw_max(sc);
    }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax), false, false);
    tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));  // max over lanes l and l ^ 32
    // the running max moves only when a score exceeds it by more than
    // kMaxSlack: probabilities stay <= 2^kMaxSlack and O is rescaled rarely
    const bool grow = tmax > m + kMaxSlack;
    if (__any(grow)) {
      asm volatile("" ::: "memory");
      const float mnew = grow ? tmax : m;
      const float alpha = (mnew == kNegInf) ? 1.f : fast_exp2(m - mnew);
      m = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < Mma::ND; ++db) mma.o[db] *= alpha;
    }
    const float muse = (m == kNegInf) ? 0.f : m;
    if (use_cap && poly) {
      // exponent = (c / 2) u (1 - y^2 / 3), y^2 = u^2 / (4 log2(e)^2)
      constexpr float k2 = 0.12011325347955035f;  // 1 / (4 log2(e)^2)
      const float a0 = 0.5f * cap, a1 = -a0 * k2 / 3.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float u = sc[q >> 1][8 * (q & 1) + i], w2 = u * u;
          pb[q][i] = (f16)fast_exp2(fmaf(u, fmaf(w2, a1, a0), -muse));
        }
    } else if (use_cap && plain) {
      const float c0 = capA - muse;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          pb[q][i] = (f16)fast_exp2(c0 - capB * fast_rcp(fast_exp2(sc[q >> 1][8 * (q & 1) + i]) + 1.f));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[q][i] = (f16)fast_exp2(sc[q >> 1][8 * (q & 1) + i] - muse);
    }
    const half2v one2 = {(f16)1.f, (f16)1.f};
    float ps[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ps[q] = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ps[q] = __builtin_amdgcn_fdot2(half2v{pb[q][2 * j], pb[q][2 * j + 1]}, one2, ps[q], false);
    }
    lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);
  };

  // ---- phases ------------------------------------------------------------------
  // M(s): copies of K(s + 1) and V(s) into LDS; PV(s - 1); scores of tile s.
  // Buffers alternate with the parity of s (compile time here).
  constexpr int kLook = 4;  // MFMA pairs whose operand reads are in flight
  const uint32_t kaddr = lds_byte(K0) + 2u * (uint32_t)((lane & 31) * L::KS + 8 * (lane >> 5));
  // M(s) for s >= 1 (parity O of s): copies of K(s + 1) and V(s), then PV(s - 1)
  // and the scores of tile s.  At s = n_tiles the scores read a stale K buffer
  // and are never used (one MFMA mix for every M phase keeps the code, and the
  // register allocation, to a single variant).
  // the copies of an M phase: K(tk) into kdst and V(tv) into vdst (each when
  // its flag is set); copy i < MK is this wave's K slot i, the others its V
  // slots
  struct Copies {
    const f16* ksrc; const f16* vsrc;
    f16* kdst; f16* vdst;
    int klast, vlast;
    bool kon, von, kwhole, vwhole;
  };
  auto plan = [&](bool kon, int tk, f16* kdst, bool von, int tv, f16* vdst) {
    Copies c{};
    c.kon = kon;
    c.von = von;
    c.kdst = kdst;
    c.vdst = vdst;
    if (kon) {
      const TileRange r = w.tile(p, tk);
      c.klast = min(max(r.start, r.lim - 1), p.kv_rows - 1) - r.start;
      c.ksrc = kg + (int64_t)r.start * p.k_j;
      c.kwhole = c.klast == BN - 1;
    }
    if (von) {
      const TileRange r = w.tile(p, tv);
      c.vlast = min(max(r.start, r.lim - 1), p.kv_rows - 1) - r.start;
      c.vsrc = vg + (int64_t)r.start * p.k_j;
      c.vwhole = c.vlast == BN - 1;
    }
    return c;
  };
  auto copy = [&](const Copies& c, auto ic) {
    constexpr int i = decltype(ic)::value;
    if constexpr (i < MK) {
      constexpr int u = i;
      if (c.kon && wave + NW * u < L::NKI) {
        int off = koff[u];
        if (!c.kwhole) {
          int rr, col;
          k_slot(u, rr, col);
          off = min(rr, c.klast) * kj + col;
        }
        lds_dma16(c.ksrc, 2u * (uint32_t)off, lds_byte(c.kdst + 512 * (wave + NW * u)));
      }
    } else {
      constexpr int u = i - MK;
      if (c.von && wave + NW * u < L::NVI) {
        int off = voff[u];
        if (!c.vwhole) {
          int rr, col;
          v_slot(u, rr, col);
          off = min(rr, c.vlast) * kj + col;
        }
        lds_dma16(c.vsrc, 2u * (uint32_t)off, lds_byte(c.vdst + 512 * (wave + NW * u)));
      }
    }
  };
  auto phase_m = [&](auto odd, int s) {
    constexpr bool O = decltype(odd)::value;
    const Copies c = plan(s + 1 < n_tiles, s + 1, O ? K0 : K1, s < n_tiles, s, O ? V1 : V0);
    if (s <= n_tiles)
      mphase<HP, O ? 0 : 1, O ? 1 : 0, true, true, kLook, MK + MV>(mma.o, sc, vaddr, kaddr, pb, mma.qf,
                                                                 [&](auto ic) { copy(c, ic); });
    // the phase's MFMA results are read after the barrier: wait for them here
    mfma_result_fence();
  };
  // end of a phase: the copies a wave issued have landed (except after an M
  // phase, whose copies stay in flight through the next V phase), then the
  // workgroup barrier
  auto end_phase = [&](bool wait_copies) {
    if (wait_copies) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  };
  if (n_tiles > 0) load_k(0, K0);
  end_phase(true);
  if (grp == 1) end_phase(true);  // the second group runs one phase behind
  // M(0): copies of K(1) and V(0), scores of tile 0
  if (n_tiles > 0) {
    const Copies c = plan(1 < n_tiles, 1, K1, true, 0, V0);
    mphase<HP, 1, 0, false, true, kLook, MK + MV>(mma.o, sc, vaddr, kaddr, pb, mma.qf,
                                                 [&](auto ic) { copy(c, ic); });
  }
  mfma_result_fence();
  end_phase(false);
  for (int s = 0; s < n_steps; s += 2) {
    if (s < n_tiles) softmax(s);  // V(s)
    end_phase(true);
    phase_m(std::true_type{}, s + 1);
    end_phase(false);
    if (s + 1 < n_tiles) softmax(s + 1);  // V(s + 1)
    end_phase(true);
    phase_m(std::false_type{}, s + 2);
    end_phase(false);
  }
  if (grp == 0) end_phase(true);

  // ---- normalise into LDS; the stores go out with the next round's loads ----
  mfma_result_fence();
  if (!live || !w.wave_rows) continue;
  lsum += shfl_xor(lsum, 32);
  bool has_sink = false;
  float sg = 0.f;
  if (p.sink != nullptr) {
    has_sink = true;
    sg = kLog2e * to_f32(static_cast<const f16*>(p.sink)[h]);
  } else if (p.smooth == 1) {
    has_sink = true;
  }
  float inv;
  if (lsum == 0.f) {
    inv = 0.f;
  } else if (has_sink) {
    const float M2 = fmaxf(m, sg);
    const float den = lsum * fast_exp2(m - M2) + fast_exp2(sg - M2);
    inv = fast_exp2(m - M2) / den;
  } else {
    inv = 1.f / lsum;
  }
  {
    f16* stage = V0 + wave * 32 * HP;
    const int r = lane & 31;
#pragma unroll
    for (int db = 0; db < Mma::ND; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int c = 4 * db + gq;  // 16-byte chunk of dims 32 db + 8 gq ..
        const half4v v = {(f16)(mma.o[db][4 * gq] * inv), (f16)(mma.o[db][4 * gq + 1] * inv),
                          (f16)(mma.o[db][4 * gq + 2] * inv), (f16)(mma.o[db][4 * gq + 3] * inv)};
        *reinterpret_cast<half4v*>(stage + r * HP + 8 * (c ^ (r & OSW)) + 4 * (lane >> 5)) = v;
      }
  }
  if (lane == 0) {
    f16* og = static_cast<f16*>(p.out);
    s_pend_rows[wv] = min(32, w.wg_rows_end - w.wrow0);
    s_pend_base[wv] = og + (int64_t)b * p.o_b + (int64_t)w.wrow0 * p.o_s + (int64_t)h * p.o_h;
  }
  }
  {
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) & 3;
    const int grp = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) >> 2;
    store_pending(lds + grp * GL + 2 * L::KTILE + wave * 32 * HP);
  }
}

template <typename T, int HP, int BN, int MODE, bool SOFTCAP = false>
hipError_t launch_mode(const FlashParams& p, dim3 grid, int nw, hipStream_t s) {
  if (nw == 4) launch_kernel((flash_kernel<T, HP, BN, MODE, 4, SOFTCAP>), grid, dim3(256), 0, s, p);
  else if (nw == 2) launch_kernel((flash_kernel<T, HP, BN, MODE, 2, SOFTCAP>), grid, dim3(128), 0, s, p);
  else launch_kernel((flash_kernel<T, HP, BN, MODE, 1, SOFTCAP>), grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

// Two items of the (gx, gy, gz) item grid per eight-wave workgroup.
template <int HP, int MODE, bool SOFTCAP = false>
hipError_t launch_pp(const FlashParams& p, dim3 grid, hipStream_t s) {
  static_assert(MODE == kDense, "the ping-pong kernel serves dense prompts");
  // one workgroup per CU at most, each looping over pairs of items (pairs of
  // head groups)
  const int pairs = (int)grid.x * (((int)grid.y + 1) / 2) * (int)grid.z;
  const int wgs = std::min(pairs, cu_count());
  if (wgs <= 0) return hipSuccess;
  launch_kernel((flash_pp_kernel<HP, MODE, SOFTCAP>), dim3(wgs), dim3(512), 0, s, p,
                     (int)grid.x, (int)grid.y, (int)grid.z);
  return hipGetLastError();
}

template <typename T, int HP, int BN>
hipError_t launch_flash_t(const FlashParams& p, dim3 grid, hipStream_t s) {
  // dense f16 prompts with heads up to 128 run on the ping-pong kernel (four
  // waves of 32 rows per item).  Varlen items (a packed sequence's row block,
  // 32 to 512 keys) are too short for its per-round start: the four-wave
  // flash kernel, many workgroups per CU, runs them faster (54-58 us against
  // 64-65 us on the 64-sequence packed batch, the same device)
  constexpr bool kPipe = std::is_same<T, f16>::value && BN == 64 && HP <= 128;
  switch (p.mode) {
    case kDense: {
      const int nw = p.rows_per_wg / 32 * p.heads_per_wg;
      if constexpr (kPipe) {
        if (nw != 4) return hipErrorInvalidValue;
        if (p.softcap > 0.f) return launch_pp<HP, kDense, true>(p, grid, s);
        return launch_pp<HP, kDense, false>(p, grid, s);
      } else {
        if (nw != 4) return hipErrorInvalidValue;
        if (p.softcap > 0.f) launch_kernel((flash_kernel<T, HP, BN, kDense, 4, true>), grid, dim3(256), 0, s, p);
        else launch_kernel((flash_kernel<T, HP, BN, kDense, 4, false>), grid, dim3(256), 0, s, p);
        return hipGetLastError();
      }
    }
    case kCsr: {
      const int nw = (p.rows_per_wg + 31) / 32;
      return launch_mode<T, HP, BN, kCsr>(p, grid, nw >= 4 ? 4 : (nw == 2 ? 2 : 1), s);
    }
    default:
      launch_kernel((flash_kernel<T, HP, BN, kVarlen, 4, false>), grid, dim3(256), 0, s, p);
      return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_flash(DType dt, int hp, const FlashParams& p, int gx, int gy, int gz,
                        hipStream_t s) {
  dim3 grid(gx, gy, gz);
  if (gx == 0 || gy == 0 || gz == 0) return hipSuccess;
  // code caches are read by the float32 dense kernel only
  if (p.qbits != 0 && (dt != DType::F32 || p.mode != kDense || (p.qbits != 8 && p.qbits != 4)))
    return hipErrorInvalidValue;
  if (dt == DType::F16) {
    if (hp == 64) return launch_flash_t<f16, 64, 64>(p, grid, s);
    if (hp == 128) return launch_flash_t<f16, 128, 64>(p, grid, s);
    return launch_flash_t<f16, 256, 64>(p, grid, s);
  }
  if (hp == 64) return launch_flash_t<float, 64, 32>(p, grid, s);
  if (hp == 128) return launch_flash_t<float, 128, 32>(p, grid, s);
  return launch_flash_t<float, 256, 32>(p, grid, s);
}

}  // namespace kvattn
