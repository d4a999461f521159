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
//     (PackedAttention page, Inputs table: weights columns are [Q all heads |
//     K all heads | V all heads]) as an MFMA GEMM with 128x128 output tiles,
//     LDS double buffering and the bias added in the epilogue.  The weights
//     are row-major [D][cols], so the B operand (k-contiguous per lane) is
//     read from the LDS tile with ds_read_b64_tr_b16.
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
constexpr int BM = 128, BNC = 128;
// k depth of a tile (64 measured slower for f16: three waves per SIMD become two)
template <typename T> struct GemmBK { static constexpr int value = 32; };
template <> struct GemmBK<float> { static constexpr int value = 32; };

typedef __fp16 lds_half4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
__device__ __forceinline__ half4v lds_tr16(const f16* ptr) {
  auto r = __builtin_amdgcn_ds_read_tr16_b64_v4f16(
      (__attribute__((address_space(3))) lds_half4*)(ptr));
  return half4v{(f16)r[0], (f16)r[1], (f16)r[2], (f16)r[3]};
}

template <typename T> struct GemmTile;

template <> struct GemmTile<f16> {
  static constexpr int BK = GemmBK<f16>::value;
  static constexpr int AS = BK + 8;     // A tile row stride (elements), rows = M
  // B tile row stride (elements), rows = K: 64 modulo 256 bytes, so the four
  // rows of one transposing read (64 bytes each) tile the banks exactly
  static constexpr int BS = BNC + 32;
  static constexpr int CH = 8;
  // acc[i][j]: 32x32 output block (i: m, j: n) of this wave's 64x64
  __device__ static void step(const f16* As, const f16* Bs, int wm, int wn, int lane,
                              float16v (&acc)[2][2]) {
    const int G = lane >> 4, t = lane & 15, c = t & 3, ir = t >> 2;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      half8v a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const half8v*>(As + (64 * wm + 32 * i + (lane & 31)) * AS +
                                                16 * ks + 8 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const f16* base = Bs + (16 * ks + 8 * (G >> 1) + ir) * BS + 64 * wn + 32 * j + 16 * (G & 1) + 4 * c;
        half4v lo = lds_tr16(base);
        half4v hi = lds_tr16(base + 4 * BS);
        b[j] = half8v{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
  }
};

template <> struct GemmTile<float> {
  static constexpr int BK = GemmBK<float>::value;
  static constexpr int AS = BK + 4;
  static constexpr int BS = BNC + 4;
  static constexpr int CH = 4;
  __device__ static void step(const float* As, const float* Bs, int wm, int wn, int lane,
                              float16v (&acc)[2][2]) {
    const int hi = lane >> 5, l32 = lane & 31;
#pragma unroll 4
    for (int ks = 0; ks < BK / 2; ++ks) {
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = As[(64 * wm + 32 * i + l32) * AS + 2 * ks + hi];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = Bs[(2 * ks + hi) * BS + 64 * wn + 32 * j + l32];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x2f32(a[i], b[j], acc[i][j]);
    }
  }
};

template <typename T>
__global__ __launch_bounds__(256) void qkv_gemm_kernel(GemmParams p) {
  using G = GemmTile<T>;
  constexpr int AS = G::AS, BS = G::BS, CH = G::CH, BK = G::BK;
  constexpr int A_EL = BM * AS, B_EL = BK * BS;
  constexpr int A_CH = BM * BK / CH, B_CH = BK * BNC / CH;   // 16-byte chunks per tile
  constexpr int CPT = (A_CH + B_CH) / 256;
  __shared__ __attribute__((aligned(16))) T lds[2 * (A_EL + B_EL)];
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

  uint4v stage[CPT];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int idx = tid + 256 * u;
      if (idx < A_CH) {
        const int r = idx / (BK / CH), kc = (idx % (BK / CH)) * CH;
        const int gm = min(m0 + r, p.M - 1), gk = k0 + kc;
        stage[u] = (gk < p.K) ? *reinterpret_cast<const uint4v*>(X + (int64_t)gm * p.K + gk)
                              : uint4v{0u, 0u, 0u, 0u};
      } else {
        const int bi = idx - A_CH;
        const int r = bi / (BNC / CH), nc = (bi % (BNC / CH)) * CH;
        const int gk = k0 + r, gn = n0 + nc;
        stage[u] = (gk < p.K && gn < p.Ncol)
                       ? *reinterpret_cast<const uint4v*>(W + (int64_t)gk * p.Ncol + gn)
                       : uint4v{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store = [&](int buf) {
    T* As = lds + buf * (A_EL + B_EL);
    T* Bs = As + A_EL;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int idx = tid + 256 * u;
      if (idx < A_CH) {
        const int r = idx / (BK / CH), kc = (idx % (BK / CH)) * CH;
        *reinterpret_cast<uint4v*>(As + r * AS + kc) = stage[u];
      } else {
        const int bi = idx - A_CH;
        const int r = bi / (BNC / CH), nc = (bi % (BNC / CH)) * CH;
        *reinterpret_cast<uint4v*>(Bs + r * BS + nc) = stage[u];
      }
    }
  };

  float16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = float16v{};

  const int nk = (p.K + BK - 1) / BK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * BK);
    const T* As = lds + buf * (A_EL + B_EL);
    G::step(As, As + A_EL, wm, wn, lane, acc);
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

  mfma_result_fence();
  T* Y = static_cast<T*>(p.y);
  const T* bias = static_cast<const T*>(p.bias);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + 64 * wn + 32 * j + (lane & 31);
    if (n >= p.Ncol) continue;
    const float bv = to_f32(bias[n]);
    // row-major Y[m][n], or head-major Y[n / hd][m][n % hd] for head size hd
    int64_t col, mstride;
    if (p.head_dim > 0) {
      col = (int64_t)(n / p.head_dim) * p.M * p.head_dim + n % p.head_dim;
      mstride = p.head_dim;
    } else {
      col = n;
      mstride = p.Ncol;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (m < p.M) Y[col + (int64_t)m * mstride] = from_f32<T>(acc[i][j][e] + bv);
      }
  }
}

}  // namespace

hipError_t launch_packed_sched(const PackedSchedParams& p, hipStream_t s) {
  size_t shmem = sizeof(int32_t) * (3 * (size_t)p.B + 1);
  hipLaunchKernelGGL(packed_sched_kernel, dim3(1), dim3(256), shmem, s, p);
  return hipGetLastError();
}

hipError_t launch_qkv_gemm(DType dt, const GemmParams& p, hipStream_t s) {
  if (p.M == 0 && !p.with_sched) return hipSuccess;
  const int tiles = ((p.M + BM - 1) / BM) * ((p.Ncol + BNC - 1) / BNC) + (p.with_sched ? 1 : 0);
  if (dt == DType::F16)
    hipLaunchKernelGGL(qkv_gemm_kernel<f16>, dim3(tiles), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(qkv_gemm_kernel<float>, dim3(tiles), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvattn
