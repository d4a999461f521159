// Internal interface between the C ABI (api.cpp) and the HIP kernels.
// Parameter blocks are plain structs passed by value to the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvattn {

// Measurement hook: events the next kernel launch takes its start and stop
// times on (the dispatch's own timestamps), or null.  Thread-local, set by the
// C ABI around the launch it profiles.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();

// Launch a kernel on stream s (errors are left for hipGetLastError).  When
// launch_events() holds events, this launch records its start and stop on
// them and clears them.
template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                          Args... args) {
  LaunchEvents& ev = launch_events();
  if (ev.start != nullptr) {
    const hipEvent_t start = ev.start, stop = ev.stop;
    ev = LaunchEvents{};
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, start, stop, 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
  }
}

// Q8: float32 activations over an int8 key/value cache (decode, and the
// byte copies of such a cache)
enum class DType : int { F32 = 1, F16 = 2, Q8 = 3, Q4 = 4 };

// ---------------------------------------------------------------------------
// K1 prep: per new token, optional per-head RMSNorm and rotary on the query
// heads (written to a query workspace) and on the key heads (written with the
// values into the cache rows at the token's absolute position).
// ---------------------------------------------------------------------------
struct PrepParams {
  const void* q;            // (B, S, q_stride) storage T; heads at q_off + h*H
  const void* k;            // (B, S, k_stride)
  const void* v;            // (B, S, v_stride)
  int64_t q_stride, k_stride, v_stride;   // elements per token row
  int64_t q_off, k_off, v_off;            // element offset of head 0 in a row
  void* q_out;              // (B, S, N*H) transformed queries, or null
  void* kc;                 // key cache (B, kvN, cap, H)
  void* vc;                 // value cache
  const void* q_norm;       // (H) or null
  const void* k_norm;       // (H) or null
  float eps;
  const void* cos;          // (rot_rows, rot_half) or null
  const void* sin;
  int rot_half;             // rotary pairs per head (r/2)
  int rot_rows;             // rows of the cos/sin tables
  int interleaved;          // 1: pairs (2i, 2i+1); 0: pairs (i, i + r/2)
  const int32_t* lens;      // per-batch lengths (device)
  int pos_mode;             // 0: none (past 0); 1: past = lens[b] + 1 - S; 2: past = lens[b] - S
  int B, S, N, kvN, H, cap;
  int write_q;              // 1: write transformed queries
  int write_kv;             // 1: append k, v into the caches
  int win_cap;              // > 0: sliding-window cache of this capacity (rows from window_geom)
  // quantised caches (T = float32, write_kv only): the new keys and values
  // are stored as codes in kq/vq (rows of H int8, or H/2 bytes of two
  // +8-biased nibbles, capacity qcap) and, unless kc/vc are null, as
  // code * scale in kc/vc
  int bits;                 // 0: float caches; 8 or 4
  void* kq; void* vq;
  int qcap;
  const float* k_scale; const float* v_scale;
  int k_scale_pc, v_scale_pc;  // 1: kvN*H per-channel scales; 0: one scale
  // a prompt's present cache in its own float type (write_kv only): the new
  // rows also go to kx/vx (B, kvN, xcap, H), float32 when x_f32 else
  // float16, each rounded once from the float32 result; null = none
  void* kx; void* vx;
  int xcap, x_f32;
};

// Sliding-window cache of capacity cap (GroupQueryAttention page, Attributes
// table: sliding_window_cache): the buffer holds the most recent tokens,
// oldest first.  For a sample with `total` tokens seen (the S new ones
// included): `held` rows before the call, `drop` rows evicted from the front,
// `fill` rows after the append, and the absolute position of row 0.
struct WindowGeom {
  int held, drop, fill, first;
};
__host__ __device__ inline WindowGeom window_geom(int total, int S, int cap) {
  WindowGeom g;
  const int before = total - S < 0 ? 0 : total - S;
  g.held = before < cap ? before : cap;
  g.drop = g.held + S - cap > 0 ? g.held + S - cap : 0;
  g.fill = g.held - g.drop + S;
  g.first = total - g.fill;
  return g;
}

// Move the rows of each (sample, kv head) slab that survive the eviction to
// the front of the buffer (rows [drop, held) to [0, held - drop)).
struct WindowShiftParams {
  void* kc; void* vc;               // (B, kvN, cap, row_bytes), shifted in place
  const int32_t* lens;              // seqlens_k (total = lens[b] + 1)
  int B, kvN, S, cap;
  int row_bytes;                    // bytes per cache row: a multiple of 4, at most 1024
};

// Copy the live past rows [0, past_b) into a separate present buffer, or,
// for a sliding-window cache (win_cap > 0), the rows that survive the
// eviction, [drop, held), to [0, held - drop) (window_geom with capacity
// win_cap; held never beyond past_seq).
struct CopyPastParams {
  const void* pk; const void* pv;   // (B, kvN, past_seq, H)
  void* ck; void* cv;               // (B, kvN, cap, H)
  const int32_t* lens;              // seqlens_k
  int B, kvN, H, S, past_seq, cap;
  int win_cap;
};

// ---------------------------------------------------------------------------
// K3 decode: one query token per sample against a BNSH cache, split over the
// key axis with a log-sum-exp combine done by the last pair of each unit.
// ---------------------------------------------------------------------------
struct DecodeParams {
  const void* q;            // (B, N*H)
  const void* k_new;        // (B, kvN*H) token key row, or null (no append)
  const void* v_new;
  void* kc;                 // (B, kvN, cap, H)
  void* vc;
  const void* q_norm;       // (H) or null
  const void* k_norm;
  float eps;
  const void* cos;          // (rows, H/2) NeoX rotary tables or null
  const void* sin;
  int rot_rows;             // rows of the rotary tables
  const void* bias;         // additive score bias or null: bias[b*bias_sb + h*bias_sh + j]
  int64_t bias_sb, bias_sh;
  int bias_cols;            // columns of the bias (keys beyond get no bias)
  const int32_t* mask;      // (B, mask_cols) int32 or null; 0 adds mask_filter
  int mask_cols;
  float mask_filter;
  const void* sink;         // (N) or null
  int smooth;               // 1: zero sink when no sink tensor
  const int32_t* lens;      // device lengths
  int len_mode;             // 0: n_b = lens[b] + 1; 1: n_b = lens[0] + 1; 2: n_b = host_n; 3: n_b = lens[b]
  int host_n;
  int window;               // >= 0: keys j >= (n_b - 1) - window
  int win_cap;              // > 0: sliding-window cache of this capacity (len_mode 0 only)
  void* out;                // (B, N*H)
  void* qk;                 // (B, N, 1, host_n) scores after mask, or null
  int qk_f32;               // qk element type: 1 float32, 0 float16 (either, whatever T is)
  float* part;              // (waves / 2, hpw, HP + 4) per-pair partials: m, l, -, -, o[HP]
  int* counters;            // (B * kvN * head_groups) arrivals per unit: zero on entry, left zero
  int split;                // 0: every unit gets one pair (no counters are touched)
  int B, N, kvN, H, cap;
  float scale, softcap;
  int head_groups;          // query-head groups of <= 16 per kv head
  int hpw;                  // partial records per wave: min(16, N / kvN)
  int waves;                // waves in the grid (a multiple of 4, >= B * kvN * head_groups)
  // int8 caches (DType::Q8): cache value = code * scale; the key scales are
  // folded into the query, the value scales applied to each pair's output
  const float* k_scale; const float* v_scale;
  int k_scale_pc, v_scale_pc;  // 1: kvN*H per-channel scales; 0: one scale
  // cache slabs: unit kv index k reads slab b * (kvN / kv_div) + k / kv_div
  // (0 = 1: one slab per unit kv index)
  int kv_div;
  // CSR block keys (SparseAttention token generation, len_mode 3): a unit is
  // one query head h (kvN = N); its keys are the blocks of CSR row
  // (n_b - 1) / block of layout h mod num_layout, in row order; a key is
  // visible iff its row is <= n_b - 1.  Null csr_rp: keys [kstart, n_b).
  const int32_t* csr_rp; const int32_t* csr_cols;
  int64_t rp_stride, cols_stride;
  int num_layout, block, max_blocks;
};

// ---------------------------------------------------------------------------
// K2 flash attention (dense causal/window, CSR block-sparse, packed varlen).
// ---------------------------------------------------------------------------
enum FlashMode : int { kDense = 0, kCsr = 1, kVarlen = 2 };

// Compute units of the current device (cached per device).
int cu_count();

struct FlashParams {
  const void* q;            // queries, element (b, s, h, d) at q_b*b + q_s*s + q_h*h + d
  int64_t q_b, q_s, q_h;
  const void* kc;           // keys, element (b, kvh, j, d) at k_b*b + k_h*kvh + k_j*j + d
  const void* vc;
  int64_t k_b, k_h, k_j;
  void* out;                // element (b, s, h, d) at o_b*b + o_s*s + o_h*h + d
  int64_t o_b, o_s, o_h;
  const void* bias;         // dense: bias[b*sb + h*sh + s*ss + j]; varlen: padded coords
  int64_t bias_sb, bias_sh, bias_ss;
  int bias_cols;            // key columns of the bias (keys beyond get no bias)
  const void* sink;         // (N) or null
  int smooth;
  const int32_t* lens;      // dense: seqlens_k (n_b = lens[b] + 1); varlen: per-sequence [start, end)
  int has_past;             // dense: 1 => past_b = n_b - S
  int win_cap;              // dense: > 0 => sliding-window cache of this capacity
  int causal;
  int window;
  // CSR
  const int32_t* rp; const int32_t* cols; int64_t rp_stride, cols_stride;
  int num_layout, block;    // block = sparse block size
  int max_blocks;           // column entries are clamped into [0, max_blocks)
  const int32_t* key_total; // sparse: per-batch key totals
  // varlen
  const int32_t* token_offset; int pad_seq;
  const int32_t* work;      // varlen work list: work[0] = count, then (b, tile) pairs
  int kv_rows;              // rows addressable in the K/V buffers (per sample / total)
  int B, S, N, kvN, H;
  float scale, softcap;
  int rows_per_wg;          // query rows per workgroup
  int heads_per_wg;         // query heads per workgroup (GQA grouping)
  int mode;
  // query preparation at load (dense and CSR modes): per-head RMSNorm with
  // q_norm (or null), rotary of the first 2 * rot_half dims with the cos/sin
  // tables (or null) at position past + row, NeoX pairs (i, i + rot_half) or
  // interleaved pairs (2i, 2i + 1)
  const void* q_norm;
  float eps;
  const void* cos;
  const void* sin;
  int rot_half, rot_rows, interleaved;
  // quantised caches (float32 queries, dense mode): kc/vc hold codes, rows of
  // H int8 (qbits 8) or H/2 bytes of two +8-biased nibbles, even dim low
  // (qbits 4), at the element strides above; each element is code * scale
  // (per-tensor scale, or per kv head and dim when *_pc)
  int qbits;
  const float* qk_scale; const float* qv_scale;
  int qk_pc, qv_pc;
};

// ---------------------------------------------------------------------------
// K5 packed: schedule + QKV projection GEMM.
// ---------------------------------------------------------------------------
struct PackedSchedParams {
  const int32_t* cum;       // (B + 1) as given
  int32_t* bounds;          // (B, 2) sanitised [start, end) per sequence
  int32_t* work;            // work[0] = count, then (b, tile) pairs, longest sequences first
  int32_t* tok_seq;         // optional (T): owning sequence per packed token
  int32_t* tok_pos;         // optional (T): position inside the sequence
  int B, T, pad_seq, tile;  // tile = query rows per attention workgroup
};

struct GemmParams {
  const void* x;            // (M, K) row-major
  const void* w;            // (K, Ncol) row-major
  const void* bias;         // (Ncol)
  void* y;                  // (M, Ncol) row-major
  int M, K, Ncol;
  int head_dim;             // > 0: write Y head-major, (Ncol / head_dim, M, head_dim)
  int with_sched;           // 1: workgroup 0 also builds `sched` (B <= kGemmSchedMaxB)
  PackedSchedParams sched;
};
// most sequences the GEMM's extra workgroup can schedule in its LDS
constexpr int kGemmSchedMaxB = 3000;

// Launchers (defined in the .hip sources).  Each returns hipSuccess or the
// launch error.
hipError_t launch_prep(DType dt, const PrepParams& p, hipStream_t s);
hipError_t launch_copy_past(DType dt, const CopyPastParams& p, hipStream_t s);
hipError_t launch_window_shift(const WindowShiftParams& p, hipStream_t s);
hipError_t launch_decode(DType dt, int hp, const DecodeParams& p, hipStream_t s);
hipError_t launch_flash(DType dt, int hp, const FlashParams& p, int grid_x, int grid_y,
                        int grid_z, hipStream_t s);
hipError_t launch_packed_sched(const PackedSchedParams& p, hipStream_t s);
hipError_t launch_qkv_gemm(DType dt, const GemmParams& p, hipStream_t s);

// Head-size padding used by the kernels (multiple of 64, <= 256).
inline int padded_head(int H) { return H <= 64 ? 64 : (H <= 128 ? 128 : 256); }

}  // namespace kvattn
