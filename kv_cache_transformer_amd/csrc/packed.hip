// K5: PackedAttention front end.
//
//   * schedule: from cumulative_sequence_length (sequence b owns packed
//     tokens [cum[b], cum[b+1]); PackedAttention page, Inputs table), build
//     sanitised per-sequence bounds and the attention work list of
//     (sequence, 128-row query tile) items, longest sequences first so the
//     longest work starts earliest; optionally the per-token (sequence,
//     position) map.  All integer work, on the device, so the call never
//     waits for the host.
//   * QKV projection: qkv[T, q+k+v] = input[T, D] . weights[D, q+k+v] + bias
//     (PackedAttention page, Inputs table: the weight columns hold Q for
//     every head, then K, then V) as an MFMA GEMM with the bias added in an
//     epilogue that goes through LDS so that the output is stored in 16-byte
//     chunks.  f16: 256x128 output tiles, both operands copied from memory
//     straight into three LDS stages; float32: 128x128 tiles, LDS double
//     buffering fed from register stages a few tiles ahead.  The weights are
//     row-major [D][cols], so the B operand (k-contiguous per lane) is read
//     from the LDS tile with a transposing read (f16: ds_read_b64_tr_b16).
#include <type_traits>
#include <utility>

#include "device_common.hpp"
#include "kvattn_internal.hpp"

namespace kvattn {
namespace {

// ---------------------------------------------------------------------------
// schedule
// ---------------------------------------------------------------------------
// One workgroup builds the schedule; sh holds 3 * B + 1 ints.
__device__ void build_schedule(const PackedSchedParams& p, int32_t* sh) {
  int32_t* len = sh;               // B
  int32_t* order = sh + p.B;       // B: sequence at each rank
  int32_t* off = sh + 2 * p.B;     // B + 1: first item of each rank
  const int tid = threadIdx.x;
  for (int b = tid; b < p.B; b += blockDim.x) {
    int start = min(max(p.cum[b], 0), p.T);
    int end = min(max(p.cum[b + 1], start), min(p.T, start + p.pad_seq));
    p.bounds[2 * b] = start;
    p.bounds[2 * b + 1] = end;
    len[b] = end - start;
  }
  __syncthreads();
  for (int b = tid; b < p.B; b += blockDim.x) {
    const int lb = len[b];
    int rank = 0;
    for (int o = 0; o < p.B; ++o) rank += (len[o] > lb) || (len[o] == lb && o < b);
    order[rank] = b;
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int k = 0; k < p.B; ++k) {
      off[k] = acc;
      acc += (len[order[k]] + p.tile - 1) / p.tile;
    }
    off[p.B] = acc;
    p.work[0] = acc;
  }
  __syncthreads();
  for (int k = tid; k < p.B; k += blockDim.x) {
    const int b = order[k];
    const int n = off[k + 1] - off[k];
    for (int t = 0; t < n; ++t) {
      p.work[1 + 2 * (off[k] + t)] = b;
      p.work[2 + 2 * (off[k] + t)] = t;
    }
  }
  if (p.tok_seq != nullptr) {
    for (int b = 0; b < p.B; ++b) {
      const int start = min(max(p.cum[b], 0), p.T);
      const int end = min(max(p.cum[b + 1], start), min(p.T, start + p.pad_seq));
      for (int t = start + tid; t < end; t += blockDim.x) {
        p.tok_seq[t] = b;
        p.tok_pos[t] = t - start;
      }
    }
  }
}

__global__ __launch_bounds__(256) void packed_sched_kernel(PackedSchedParams p) {
  extern __shared__ int32_t sh[];
  build_schedule(p, sh);
}

// ---------------------------------------------------------------------------
// QKV projection GEMM
// ---------------------------------------------------------------------------
constexpr int BNC = 128;
// register stages of the operand prefetch (tiles in flight while one is used)
constexpr int kGemmStages = 3;
// buffer resource word 3 for raw 32-bit buffer accesses (gfx9 family)
constexpr int kGemmBufferFormat = 0x00020000;
// f16 GEMM: 32-row blocks per wave, waves across the columns (64 columns
// each), LDS stages and workgroups per CU (workgroup tile 256 x 128)
constexpr int kGemmMbF16 = 4;
constexpr int kGemmNwnF16 = 2;
constexpr int kGemmStagesF16 = 3;
constexpr int kGemmOccF16 = 2;

// Calls f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>).
template <int N, typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for_int(F&& f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

typedef __fp16 lds_half4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
__device__ __forceinline__ half4v lds_tr16(const f16* ptr) {
  auto r = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (__attribute__((address_space(3))) lds_half4*)(ptr));
  return half4v{(f16)r[0], (f16)r[1], (f16)r[2], (f16)r[3]};
}

// four consecutive elements stored at once
template <typename T> struct Quad4;
template <> struct Quad4<f16> {
  __device__ static void store(f16* y, const float (&v)[4]) {
    *reinterpret_cast<half4v*>(y) = half4v{(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
  }
  __device__ static void load(const f16* x, float (&v)[4]) {
    const half4v h = *reinterpret_cast<const half4v*>(x);
    for (int r = 0; r < 4; ++r) v[r] = (float)h[r];
  }
};
template <> struct Quad4<float> {
  __device__ static void store(float* y, const float (&v)[4]) {
    *reinterpret_cast<float4v*>(y) = float4v{v[0], v[1], v[2], v[3]};
  }
  __device__ static void load(const float* x, float (&v)[4]) {
    const float4v f = *reinterpret_cast<const float4v*>(x);
    for (int r = 0; r < 4; ++r) v[r] = f[r];
  }
};

template <typename T> struct GemmTile;

template <> struct GemmTile<float> {
  static constexpr int BK = 32;
  static constexpr int AS = BK + 4;
  static constexpr int BS = BNC + 4;
  static constexpr int CH = 4;
  template <int MB>
  __device__ static void step(const float* As, const float* Bs, int wm, int wn, int lane,
                              float16v (&acc)[MB][2]) {
    const int hi = lane >> 5, l32 = lane & 31;
#pragma unroll 4
    for (int ks = 0; ks < BK / 2; ++ks) {
      float a[MB], b[2];
#pragma unroll
      for (int i = 0; i < MB; ++i) a[i] = As[(32 * MB * wm + 32 * i + l32) * AS + 2 * ks + hi];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = Bs[(2 * ks + hi) * BS + 64 * wn + 32 * j + l32];
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x2f32(b[j], a[i], acc[i][j]);
    }
  }
};

// Epilogue through LDS: the transposed blocks (element e of acc[i][j] is
// m = ... + lane % 32, n = ... + 8 (e / 4) + 4 (lane / 32) + e % 4) go with
// the bias into a row-major tile, which is then stored in 16-byte chunks
// (Ncol and the head size are multiples of 8, so a chunk stays in one head).
// Cs: LDS of at least (64 MB) x (BN + 8) elements, free on entry; NT threads.
template <typename T, int MB, int BN = BNC, int NT = 256>
__device__ __forceinline__ void gemm_epilogue(const float16v (&acc)[MB][2], T* Cs, const GemmParams& p,
                                              int m0, int n0, int wm, int wn, int lane, int tid) {
  constexpr int BM = 64 * MB;
  constexpr int CS = BN + 8;  // output tile row stride (elements)
  constexpr int CH = 16 / sizeof(T);
  const T* bias = static_cast<const T*>(p.bias);
  // the bias runs of four columns, all loads issued before any is used (Ncol
  // is a multiple of 4, so a run is wholly inside or wholly past the columns;
  // a run past them reads the last one and is dropped)
  float bias4[2][4][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + 64 * wn + 32 * j + 8 * q + 4 * (lane >> 5);
      Quad4<T>::load(bias + min(n, p.Ncol - 4), bias4[j][q]);
    }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = 64 * wn + 32 * j + 8 * q + 4 * (lane >> 5);
      const bool in = n0 + nl < p.Ncol;
      float bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) bv[r] = in ? bias4[j][q][r] : 0.f;
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int ml = 32 * MB * wm + 32 * i + (lane & 31);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r] + bv[r];
        Quad4<T>::store(Cs + ml * CS + nl, v);
      }
    }
  __syncthreads();
  T* Y = static_cast<T*>(p.y);
  constexpr int CPR = BN / CH;  // chunks per tile row
  for (int c = tid; c < BM * CPR; c += NT) {
    const int r = c / CPR, cc = (c % CPR) * CH;
    const int m = m0 + r, n = n0 + cc;
    if (m >= p.M || n >= p.Ncol) continue;
    // row-major Y[m][n], or head-major Y[n / hd][m][n % hd] for head size hd
    const int64_t at = (p.head_dim > 0)
                           ? ((int64_t)(n / p.head_dim) * p.M + m) * p.head_dim + n % p.head_dim
                           : (int64_t)m * p.Ncol + n;
    *reinterpret_cast<uint4v*>(Y + at) = *reinterpret_cast<const uint4v*>(Cs + r * CS + cc);
  }
}

// float32 projection.  MB: 32-row blocks of a wave's tile; the workgroup tile
// is (64 MB) x 128 (four waves, 2 x 2).
template <typename T, int MB>
__global__ __launch_bounds__(256, 2) void qkv_gemm_kernel(GemmParams p) {
  using G = GemmTile<T>;
  constexpr int AS = G::AS, BS = G::BS, CH = G::CH, BK = G::BK;
  constexpr int BM = 64 * MB;
  constexpr int CS = BNC + 8;  // output tile row stride (elements), epilogue
  constexpr int A_EL = BM * AS, B_EL = BK * BS;
  constexpr int A_CH = BM * BK / CH, B_CH = BK * BNC / CH;   // 16-byte chunks per tile
  constexpr int CPT = (A_CH + B_CH) / 256;
  constexpr int LDS_EL = (2 * (A_EL + B_EL) > BM * CS) ? 2 * (A_EL + B_EL) : BM * CS;
  __shared__ __attribute__((aligned(16))) T lds[LDS_EL];
  static_assert(sizeof(lds) / (sizeof(int32_t)) >= 3 * kGemmSchedMaxB + 1, "schedule fits the tile LDS");

  // workgroup 0 builds the attention schedule when asked (no separate launch)
  if (p.with_sched) {
    if (blockIdx.x == 0) {
      build_schedule(p.sched, reinterpret_cast<int32_t*>(lds));
      return;
    }
  }
  const int tile = blockIdx.x - (p.with_sched ? 1 : 0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (p.Ncol + BNC - 1) / BNC;
  const int m0 = (tile / tiles_n) * BM;
  const int n0 = (tile % tiles_n) * BNC;
  const T* X = static_cast<const T*>(p.x);
  const T* W = static_cast<const T*>(p.w);

  // register stages: tile kt + 1 waits in registers for its LDS buffer while
  // tiles up to kt + NS are still in flight
  constexpr int NS = kGemmStages;
  uint4v stages[NS][CPT];
  // Operand chunks are read through buffer resources made per k step (A from
  // row m0 and column k0 on, over the tile's valid rows; B from row k0 and
  // column n0 on), at per-lane offsets fixed for the launch, so a load costs
  // no vector address arithmetic.  The range check covers the per-lane offset
  // only (not a scalar one), hence the per-step resources.  Out-of-range chunks
  // read 0: A rows past M, B rows past K.  B chunks past Ncol read the next
  // row's first columns; they only reach output columns that are never
  // stored.  A chunks past K (a partial last k step) read the next row and are
  // zeroed when written to LDS.
  static_assert(A_CH % 256 == 0 && B_CH % 256 == 0, "whole chunk rows per thread");
  constexpr int NA = A_CH / 256, NB = B_CH / 256;
  constexpr int ES = sizeof(T);
  const int rows_a = min(p.M - m0, BM);
  auto rsrc_a = [&](int k0) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(X) + (int64_t)m0 * p.K + k0, 0,
                                             (rows_a * p.K - k0) * ES, kGemmBufferFormat);
  };
  auto rsrc_b = [&](int k0) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(W) + (int64_t)k0 * p.Ncol + n0, 0,
                                             ((p.K - k0) * p.Ncol - n0) * ES, kGemmBufferFormat);
  };
  int aoff[NA], boff[NB], alds[NA], blds[NB], akc[NA];
#pragma unroll
  for (int u = 0; u < NA; ++u) {
    const int idx = tid + 256 * u;
    const int r = idx / (BK / CH), kc = (idx % (BK / CH)) * CH;
    aoff[u] = (r * p.K + kc) * ES;
    alds[u] = r * AS + kc;
    akc[u] = kc;
  }
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int bi = tid + 256 * u;
    const int r = bi / (BNC / CH), nc = (bi % (BNC / CH)) * CH;
    boff[u] = (r * p.Ncol + nc) * ES;
    blds[u] = r * BS + nc;
  }
  auto load = [&](auto st, int k0) {
    uint4v (&stage)[CPT] = stages[decltype(st)::value];
    const __amdgpu_buffer_rsrc_t ra = rsrc_a(k0), rb = rsrc_b(k0);
#pragma unroll
    for (int u = 0; u < NA; ++u)
      stage[u] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(ra, aoff[u], 0, 0));
#pragma unroll
    for (int u = 0; u < NB; ++u)
      stage[NA + u] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(rb, boff[u], 0, 0));
  };
  auto store = [&](auto st, int buf, int k0) {
    uint4v (&stage)[CPT] = stages[decltype(st)::value];
    T* As = lds + buf * (A_EL + B_EL);
    T* Bs = As + A_EL;
    if (k0 + BK > p.K) {
      const uint4v zero = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < NA; ++u)
        if (k0 + akc[u] >= p.K) stage[u] = zero;
    }
#pragma unroll
    for (int u = 0; u < NA; ++u) *reinterpret_cast<uint4v*>(As + alds[u]) = stage[u];
#pragma unroll
    for (int u = 0; u < NB; ++u) *reinterpret_cast<uint4v*>(Bs + blds[u]) = stage[NA + u];
  };

  float16v acc[MB][2];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = float16v{};

  const int nk = (p.K + BK - 1) / BK;
  // prologue: tiles 0 .. NS - 1 in flight (past the last tile: the last one
  // again), tile 0 into LDS buffer 0
  const int k_last = (nk - 1) * BK;
  static_for_int<NS>([&](auto st) { load(st, min(decltype(st)::value * BK, k_last)); });
  store(std::integral_constant<int, 0>{}, 0, 0);
  __syncthreads();
  // iteration kt: MFMAs on buffer kt & 1; tile kt + 1 (stage (kt + 1) % NS)
  // into the other buffer; tile kt + NS loads into stage kt % NS, free since
  // tile kt went to LDS
  for (int k0 = 0; k0 < nk; k0 += NS) {
    static_for_int<NS>([&](auto st) {
      constexpr int s0 = decltype(st)::value;
      const int kt = k0 + s0;
      if (kt < nk) {
        const T* As = lds + (kt & 1) * (A_EL + B_EL);
        G::template step<MB>(As, As + A_EL, wm, wn, lane, acc);
        if (kt + 1 < nk) store(std::integral_constant<int, (s0 + 1) % NS>{}, (kt + 1) & 1, (kt + 1) * BK);
        load(std::integral_constant<int, s0>{}, min((kt + NS) * BK, k_last));
        __syncthreads();
      }
    });
  }

  mfma_result_fence();
  // The last loop iteration ended with a barrier, so the stage buffers are free.
  gemm_epilogue<T, MB>(acc, lds, p, m0, n0, wm, wn, lane, tid);
}


// ---------------------------------------------------------------------------
// f16 projection with both operands copied from memory straight into LDS
// (buffer loads to LDS: no register staging, no LDS store instructions),
// a few LDS stages, the copies of tile kt + stages - 1 issued while tile kt
// is used.
// A copy instruction fills 64 consecutive 16-byte LDS slots, so the tiles are
// unpadded and the bank spread comes from XOR swizzles of the 16-byte chunks
// within a row, applied by choosing which chunk each lane copies:
//   A (rows of BK = 32 elements, 4 chunks): chunk c of row r in slot
//     c ^ swz_a(r mod 16); the 16 rows of one operand read land in 16
//     distinct slots of a 256-byte bank window (and 8 rows in 8 of a 128-byte
//     one);
//   B (rows of the tile's 64 NWN columns): chunk c of row k in slot
//     c ^ 4 (k mod 4); the eight 64-byte row pieces of one transposing read
//     cover every bank twice.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz_a(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
__device__ __forceinline__ int swz_b(int k) { return 4 * (k & 3); }

// Copy 16 bytes per lane from buffer r at per-lane byte offset voff into LDS
// at byte address lds + 16 * lane (lds uniform).  The copy is waited for
// explicitly (vmcnt), so it is a volatile statement the compiler does not
// count.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               ::"v"(voff), "s"(r), "s"(lds) : "memory");
}

// MB: 32-row blocks of a wave's tile (the tile has 64 MB rows); NWN: waves
// across the tile's columns (64 each; 2 NWN waves in all); STAGES: LDS
// stages; OCC: workgroups per CU the launch bounds ask for.
template <int MB, int NWN, int STAGES, int OCC>
__global__ __launch_bounds__(128 * NWN, OCC) void qkv_gemm_dma_kernel(GemmParams p) {
  constexpr int BK = 32, BM = 64 * MB, BN = 64 * NWN, NT = 128 * NWN, NWAVE = 2 * NWN;
  constexpr int A_EL = BM * BK, B_EL = BK * BN, ST_EL = A_EL + B_EL;   // one stage
  constexpr int CS = BN + 8;
  constexpr int LDS_EL = (STAGES * ST_EL > BM * CS) ? STAGES * ST_EL : BM * CS;
  __shared__ __attribute__((aligned(1024))) f16 lds[LDS_EL];
  static_assert(sizeof(lds) / (sizeof(int32_t)) >= 3 * kGemmSchedMaxB + 1, "schedule fits the tile LDS");
  // copy instructions (1 KB each) per wave and tile; B rows per instruction
  constexpr int DA = BM / 16 / NWAVE, DB = BN / 16 / NWAVE, BLR = BN / 8, BRI = 64 / BLR;
  static_assert(A_EL * 2 == NWAVE * DA * 1024 && B_EL * 2 == NWAVE * DB * 1024, "whole copy blocks per wave");

  // Workgroups are dealt to the eight XCDs round-robin by id; renumbered so
  // that each XCD takes a contiguous range of tiles (all column tiles of a
  // few row blocks at a time), whose input rows then stay in its L2.  Id 0
  // stays 0: the workgroup that builds the attention schedule when asked.
  const int nwg = gridDim.x, x = blockIdx.x % 8;
  int idx = blockIdx.x / 8;
  for (int y = 0; y < x; ++y) idx += (nwg - y + 7) / 8;
  if (p.with_sched) {
    if (idx == 0) {
      build_schedule(p.sched, reinterpret_cast<int32_t*>(lds));
      return;
    }
  }
  const int tile = idx - (p.with_sched ? 1 : 0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;
  const int tiles_n = (p.Ncol + BN - 1) / BN;
  const int m0 = (tile / tiles_n) * BM;
  const int n0 = (tile % tiles_n) * BN;
  const f16* X = static_cast<const f16*>(p.x);
  const f16* W = static_cast<const f16*>(p.w);
  const int rows_a = min(p.M - m0, BM);
  // Per-k-step resources (the range check covers the per-lane offset only):
  // A from row m0 and column k0 over the tile's valid rows, B from row k0 and
  // column n0.  Out-of-range chunks read 0 (A rows past M, B rows past K); B
  // chunks past Ncol reach only output columns that are never stored; A
  // chunks past K (a partial last step) read the next row and are zeroed.
  auto rsrc_a = [&](int k0) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<f16*>(X) + (int64_t)m0 * p.K + k0, 0,
                                             (rows_a * p.K - k0) * 2, kGemmBufferFormat);
  };
  auto rsrc_b = [&](int k0) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<f16*>(W) + (int64_t)k0 * p.Ncol + n0, 0,
                                             ((p.K - k0) * p.Ncol - n0) * 2, kGemmBufferFormat);
  };
  // this lane's copy slots: A block q = wave DA + a holds rows 16 q .. 16 q + 15
  // (four lanes per row); B block q = wave DB + b holds rows BRI q ..
  // BRI q + BRI - 1 (BLR lanes per row)
  const int ca = (lane & 3) ^ swz_a(lane >> 2);
  int aoff[DA], boff[DB];
#pragma unroll
  for (int a = 0; a < DA; ++a) {
    const int r = 16 * (wave * DA + a) + (lane >> 2);
    aoff[a] = (r * p.K + 8 * ca) * 2;
  }
#pragma unroll
  for (int b = 0; b < DB; ++b) {
    const int k = BRI * (wave * DB + b) + lane / BLR;
    boff[b] = (k * p.Ncol + 8 * ((lane % BLR) ^ swz_b(k))) * 2;
  }
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) f16*)lds);
  auto issue = [&](int kt, int st) {
    const __amdgpu_buffer_rsrc_t ra = rsrc_a(kt * BK), rb = rsrc_b(kt * BK);
    const uint32_t base = lds0 + 2u * (uint32_t)(st * ST_EL);
#pragma unroll
    for (int a = 0; a < DA; ++a) dma16(ra, aoff[a], base + 1024u * (uint32_t)(wave * DA + a));
#pragma unroll
    for (int b = 0; b < DB; ++b) dma16(rb, boff[b], base + 2u * A_EL + 1024u * (uint32_t)(wave * DB + b));
  };

  float16v acc[MB][2];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = float16v{};

  // operand read addresses (elements, relative to a stage): A row
  // 32 MB wm + 32 i + lane % 32 (row mod 16 = lane mod 16), chunk 2 ks + lane / 32;
  // B rows 16 ks + 8 (G / 2) + ir (+ 4), G = lane / 16, ir = lane / 4 mod 4
  const int fa = swz_a(lane & 15);
  const int G = lane >> 4, cq = lane & 3, ir = (lane >> 2) & 3;
  const int nk = (p.K + BK - 1) / BK;
  // prologue: tiles 0 .. STAGES - 2 in flight (past the last tile: the
  // last one again, into a stage nothing reads)
#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t) issue(min(t, nk - 1), t);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt % STAGES;
    // this wave's copies of tile kt are done (those of the later tiles in
    // flight may run on)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((STAGES - 2) * (DA + DB)) : "memory");
    if ((kt + 1) * BK > p.K) {
      // partial last step: A chunks past K hold the next row's elements
#pragma unroll
      for (int a = 0; a < DA; ++a)
        if (kt * BK + 8 * ca >= p.K)
          *reinterpret_cast<uint4v*>(lds + st * ST_EL + 512 * (wave * DA + a) + 8 * lane) = uint4v{0u, 0u, 0u, 0u};
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the zeros land before the barrier
    }
    asm volatile("s_barrier" ::: "memory");
    // the stage of tile kt + STAGES - 1 was read in step kt - 1, which every
    // wave has finished
    issue(min(kt + STAGES - 1, nk - 1), (kt + STAGES - 1) % STAGES);
    const f16* As = lds + st * ST_EL;
    const f16* Bs = As + A_EL;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      half8v a[MB], b[2];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        a[i] = *reinterpret_cast<const half8v*>(As + (32 * MB * wm + 32 * i + (lane & 31)) * BK +
                                                8 * ((2 * ks + (lane >> 5)) ^ fa));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int R = 16 * ks + 8 * (G >> 1) + ir;
        const int ch = 8 * wn + 4 * j + 2 * (G & 1) + (cq >> 1);
        const f16* base = Bs + R * BN + 8 * (ch ^ swz_b(R)) + 4 * (cq & 1);
        half4v lo = lds_tr16(base);
        half4v hi = lds_tr16(base + 4 * BN);
        b[j] = half8v{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(b[j], a[i], acc[i][j]);
    }
  }
  mfma_result_fence();
  // every copy has landed and every wave is past its last operand read
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  gemm_epilogue<f16, MB, BN, NT>(acc, lds, p, m0, n0, wm, wn, lane, tid);
}

}  // namespace

hipError_t launch_packed_sched(const PackedSchedParams& p, hipStream_t s) {
  size_t shmem = sizeof(int32_t) * (3 * (size_t)p.B + 1);
  launch_kernel(packed_sched_kernel, dim3(1), dim3(256), shmem, s, p);
  return hipGetLastError();
}

hipError_t launch_qkv_gemm(DType dt, const GemmParams& p, hipStream_t s) {
  if (p.M == 0 && !p.with_sched) return hipSuccess;
  const int bm = dt == DType::F16 ? 64 * kGemmMbF16 : 128;
  const int bn = dt == DType::F16 ? 64 * kGemmNwnF16 : BNC;
  const int tiles = ((p.M + bm - 1) / bm) * ((p.Ncol + bn - 1) / bn) + (p.with_sched ? 1 : 0);
  if (dt == DType::F16)
    launch_kernel((qkv_gemm_dma_kernel<kGemmMbF16, kGemmNwnF16, kGemmStagesF16, kGemmOccF16>),
                       dim3(tiles), dim3(128 * kGemmNwnF16), 0, s, p);
  else
    launch_kernel((qkv_gemm_kernel<float, 2>), dim3(tiles), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvattn
