// K1: per-token preparation of new query/key/value rows.
//
// For each new token (b, s) at absolute position p = past_b + s:
//   * query heads (when requested): optional per-head RMSNorm with
//     q_norm_weight, optional rotary, written to a query workspace in BSH
//     order (GroupQueryAttention page, Inputs table: q/k_norm_weight are
//     applied before rotary; SparseAttention page, Inputs table: cos_cache
//     width fixes the rotated dims, Attributes table: rotary_interleaved);
//   * key heads: the same transform with k_norm_weight, then written to the
//     key cache row p;
//   * value heads: copied to the value cache row p.
// Cache rows other than p are never touched, so a shared or in-place cache
// keeps every unchanged row (GroupQueryAttention page, Implementation
// variants on retaining existing cache rows).
//
// Quantised caches (GroupQueryAttention page, Attributes table: k/v_quant_type,
// kv_cache_bit_width; Inputs table: k_scale, v_scale and the int4 packing;
// float32 rows only): the transformed key and the value become codes
// clamp(rint(x / scale)) (float32 quotient) in the code cache, int8 or two
// +8-biased nibbles per byte with the even dim low (and, when a float cache
// is given, code * scale there; the prompt's attention reads the codes).
//
// One workgroup (4 waves) per token; each wave transforms one head at a
// time with its lanes spread over the head's dims.  The transformed head is
// staged in LDS so that a lane can read its rotary partner.
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "kvattn_internal.hpp"

namespace kvattn {
namespace {

constexpr int kPrepThreads = 256;

// 16 bytes of T as float (8 halves or 4 floats), and back
__device__ __forceinline__ void load8_or_4(const f16* p, float (&x)[8]) { load8_f32<f16>(p, x); }
__device__ __forceinline__ void load8_or_4(const float* p, float (&x)[4]) {
  const float4v v = *reinterpret_cast<const float4v*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = v[i];
}
__device__ __forceinline__ void store8_or_4(f16* p, const float (&x)[8]) { store8_from_f32<f16>(p, x); }
__device__ __forceinline__ void store8_or_4(float* p, const float (&x)[4]) {
  *reinterpret_cast<float4v*>(p) = float4v{x[0], x[1], x[2], x[3]};
}

// Quantised store of row element d = lane + 64u (u < 4) of head h, value y[u]:
// the code into the code cache row, code * scale into the float cache row
// when there is one.  Called by all 64 lanes of a wave (the int4 pairs meet
// by a lane shuffle).
__device__ void quant_store(const PrepParams& p, bool key, int b, int h, int crow, int lane,
                            const float (&y)[4]) {
  const int H = p.H;
  const float* sc = key ? p.k_scale : p.v_scale;
  const bool pc = (key ? p.k_scale_pc : p.v_scale_pc) != 0;
  const int64_t slab = (int64_t)b * p.kvN + h;
  float* const fc = static_cast<float*>(key ? p.kc : p.vc);
  float* deq = fc != nullptr ? fc + (slab * p.cap + crow) * H : nullptr;
  const float top = p.bits == 8 ? 127.f : 7.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = lane + 64 * u;
    int c = 0;
    if (d < H) {
      const float s = pc ? sc[(int64_t)h * H + d] : sc[0];
      c = (int)fminf(fmaxf(rintf(y[u] / s), -top - 1.f), top);
      if (deq != nullptr) deq[d] = (float)c * s;
    }
    if (p.bits == 8) {
      int8_t* codes = static_cast<int8_t*>(key ? p.kq : p.vq) + (slab * p.qcap + crow) * H;
      if (d < H) codes[d] = (int8_t)c;
    } else {
      const int cp = __shfl_xor(c, 1, 64);  // the odd partner of an even dim
      uint8_t* codes = static_cast<uint8_t*>(key ? p.kq : p.vq) + (slab * p.qcap + crow) * (H / 2);
      if (d < H && (d & 1) == 0) codes[d >> 1] = (uint8_t)((c + 8) | ((cp + 8) << 4));
    }
  }
}

// Element d of a row of the cache in its own float type (kx / vx).
__device__ __forceinline__ void store_x(const PrepParams& p, void* x, int64_t row, int d, float y) {
  const int64_t at = row * p.H + d;
  if (p.x_f32) static_cast<float*>(x)[at] = y;
  else static_cast<f16*>(x)[at] = from_f32<f16>(y);
}

template <typename T>
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(PrepParams p) {
  __shared__ float row[4][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tok = blockIdx.x;
  const int b = tok / p.S, s = tok % p.S;
  const int H = p.H;

  int past = 0;
  if (p.pos_mode == 1) past = p.lens[b] + 1 - p.S;
  else if (p.pos_mode == 2) past = p.lens[b] - p.S;
  const int pos = past + s;  // rotary position
  // cache row: the position, or after the eviction of a sliding-window cache
  const int crow = p.win_cap > 0 ? window_geom(p.lens[b] + 1, p.S, p.win_cap).fill - p.S + s : pos;

  const int nq = p.write_q ? p.N : 0;
  const int nk = p.write_kv ? p.kvN : 0;
  const int total = nq + 2 * nk;
  const T* cs = static_cast<const T*>(p.cos);
  const T* sn = static_cast<const T*>(p.sin);
  const int rpos = (cs != nullptr) ? min(max(pos, 0), p.rot_rows - 1) : 0;
  const bool row_ok = crow >= 0 && crow < p.cap;

  for (int base = 4 * (int)blockIdx.y; base < total; base += 4 * (int)gridDim.y) {
    const int item = base + wave;
    if (item < total) {
      int kind, h;  // kind 0 = query, 1 = key, 2 = value
      if (item < nq) { kind = 0; h = item; }
      else if (item < nq + nk) { kind = 1; h = item - nq; }
      else { kind = 2; h = item - nq - nk; }
      const T* src;
      if (kind == 0) src = static_cast<const T*>(p.q) + (int64_t)tok * p.q_stride + p.q_off + (int64_t)h * H;
      else if (kind == 1) src = static_cast<const T*>(p.k) + (int64_t)tok * p.k_stride + p.k_off + (int64_t)h * H;
      else src = static_cast<const T*>(p.v) + (int64_t)tok * p.v_stride + p.v_off + (int64_t)h * H;

      if (kind == 2) {
        if (row_ok) {
          bool done = false;
          if constexpr (std::is_same<T, float>::value) {
            if (p.bits != 0) {
              float y[4];
#pragma unroll
              for (int u = 0; u < 4; ++u) y[u] = (lane + 64 * u < H) ? src[lane + 64 * u] : 0.f;
              quant_store(p, false, b, h, crow, lane, y);
              done = true;
            }
          }
          if (!done) {
            T* dst = static_cast<T*>(p.vc) + (((int64_t)b * p.kvN + h) * p.cap + crow) * H;
            for (int d = lane; d < H; d += 64) dst[d] = src[d];
            if (p.vx != nullptr && crow < p.xcap)
              for (int d = lane; d < H; d += 64)
                store_x(p, p.vx, ((int64_t)b * p.kvN + h) * p.xcap + crow, d, to_f32(src[d]));
          }
        }
      } else {
        const T* nw = static_cast<const T*>(kind == 0 ? p.q_norm : p.k_norm);
        float x[4];
        float ss = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          int d = lane + 64 * u;
          x[u] = (d < H) ? to_f32(src[d]) : 0.f;
          ss += x[u] * x[u];
        }
        if (nw != nullptr) {
          ss = wave_sum_xor(ss, 1, 32);
          float r = rsqrtf(ss / (float)H + p.eps);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            int d = lane + 64 * u;
            if (d < H) x[u] *= r * to_f32(nw[d]);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) row[wave][lane + 64 * u] = x[u];
        // the row is private to this wave: a wave-scope fence orders the
        // lanes' LDS writes before the partner reads below
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          int d = lane + 64 * u;
          y[u] = x[u];
          if (cs != nullptr && d < 2 * p.rot_half) {
            int i, partner;
            float sign;
            if (p.interleaved) {
              i = d >> 1;
              partner = d ^ 1;
              sign = (d & 1) ? 1.f : -1.f;
            } else {
              i = d < p.rot_half ? d : d - p.rot_half;
              partner = d < p.rot_half ? d + p.rot_half : d - p.rot_half;
              sign = d < p.rot_half ? -1.f : 1.f;
            }
            float co = to_f32(cs[(int64_t)rpos * p.rot_half + i]);
            float si = to_f32(sn[(int64_t)rpos * p.rot_half + i]);
            // first of a pair: a*cos - b*sin; second: b*cos + a*sin
            y[u] = x[u] * co + sign * row[wave][partner] * si;
          }
        }
        if (kind == 0) {
          T* dst = static_cast<T*>(p.q_out) + ((int64_t)tok * p.N + h) * H;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            int d = lane + 64 * u;
            if (d < H) dst[d] = from_f32<T>(y[u]);
          }
        } else if (row_ok) {
          bool done = false;
          if constexpr (std::is_same<T, float>::value) {
            if (p.bits != 0) {
              quant_store(p, true, b, h, crow, lane, y);
              done = true;
            }
          }
          if (!done) {
            T* dst = static_cast<T*>(p.kc) + (((int64_t)b * p.kvN + h) * p.cap + crow) * H;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              int d = lane + 64 * u;
              if (d < H) dst[d] = from_f32<T>(y[u]);
            }
            if (p.kx != nullptr && crow < p.xcap) {
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                int d = lane + 64 * u;
                if (d < H) store_x(p, p.kx, ((int64_t)b * p.kvN + h) * p.xcap + crow, d, y[u]);
              }
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

// Keys and values only, vectorised: every lane moves one 16-byte chunk of a
// row and a group of H / CH lanes holds a whole head row, so the norm is a
// sum over the group and the rotary partner (chunk +- rot_half / CH for
// half-split pairs, the neighbouring element for interleaved pairs) comes
// from a lane of the same group.  Used when rot_half is a multiple of CH (or
// no rotary, or interleaved pairs); rows are (token, kv head) in order.
template <typename T>
__global__ __launch_bounds__(kPrepThreads) void prep_kv_kernel(PrepParams p) {
  constexpr int CH = 16 / sizeof(T);
  const int H = p.H;
  const int lpr = H / CH;                    // lanes per head row (<= 64)
  const int rows_per_wave = 64 / lpr;
  const int lane = threadIdx.x & 63;
  const int grp = lane / lpr, j = lane % lpr;
  const int64_t nrows = (int64_t)p.B * p.S * p.kvN;
  const int64_t wave0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 64;
  const int64_t wstride = (int64_t)gridDim.x * blockDim.x / 64;
  const T* cs = static_cast<const T*>(p.cos);
  const T* sn = static_cast<const T*>(p.sin);
  const T* kw = static_cast<const T*>(p.k_norm);
  const int rh = p.rot_half;
  for (int64_t w = wave0; w * rows_per_wave < nrows; w += wstride) {
    const int64_t row = w * rows_per_wave + grp;
    const bool live = grp < rows_per_wave && row < nrows;
    const int64_t rr = live ? row : 0;
    const int64_t tok = rr / p.kvN;
    const int kvh = (int)(rr % p.kvN);
    const int b = (int)(tok / p.S), s = (int)(tok % p.S);
    int past = 0;
    if (p.pos_mode == 1) past = p.lens[b] + 1 - p.S;
    else if (p.pos_mode == 2) past = p.lens[b] - p.S;
    const int pos = past + s;  // rotary position
    const int crow = p.win_cap > 0 ? window_geom(p.lens[b] + 1, p.S, p.win_cap).fill - p.S + s : pos;
    const bool row_ok = live && crow >= 0 && crow < p.cap;
    const int d0 = CH * j;
    const T* ksrc = static_cast<const T*>(p.k) + tok * p.k_stride + p.k_off + (int64_t)kvh * H + d0;
    const T* vsrc = static_cast<const T*>(p.v) + tok * p.v_stride + p.v_off + (int64_t)kvh * H + d0;
    const uint4v kraw = *reinterpret_cast<const uint4v*>(ksrc);
    const uint4v vraw = *reinterpret_cast<const uint4v*>(vsrc);
    const int64_t dst = (((int64_t)b * p.kvN + kvh) * p.cap + crow) * H + d0;
    if (row_ok) *reinterpret_cast<uint4v*>(static_cast<T*>(p.vc) + dst) = vraw;
    float x[CH];
    load8_or_4(reinterpret_cast<const T*>(&kraw), x);
    if (kw != nullptr) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < CH; ++e) ss += x[e] * x[e];
      for (int m = 1; m < lpr; m <<= 1) ss += shfl_xor(ss, m);
      const float r = rsqrtf(ss / (float)H + p.eps);
      float wv[CH];
      load8_or_4(kw + d0, wv);
#pragma unroll
      for (int e = 0; e < CH; ++e) x[e] *= r * wv[e];
    }
    if (cs != nullptr) {
      const int prow = min(max(pos, 0), p.rot_rows - 1);
      float y[CH];
      if (p.interleaved) {
#pragma unroll
        for (int e = 0; e < CH; ++e) {
          const int d = d0 + e;
          y[e] = x[e];
          if (d < 2 * rh) {
            const float c = to_f32(cs[(int64_t)prow * rh + (d >> 1)]);
            const float si = to_f32(sn[(int64_t)prow * rh + (d >> 1)]);
            y[e] = (d & 1) ? x[e] * c + x[e ^ 1] * si : x[e] * c - x[e ^ 1] * si;
          }
        }
      } else {
        const int pj = (d0 < rh) ? j + rh / CH : j - rh / CH;  // partner lane in the group
        const int src = grp * lpr + ((d0 < 2 * rh) ? pj : j);
        // the chunk's dims d0 .. d0 + CH - 1 take the consecutive table entries
        // i0 .. i0 + CH - 1 (rh is a multiple of CH): one 16-byte load each
        const bool rot_chunk = d0 < 2 * rh;
        const int i0 = rot_chunk ? (d0 < rh ? d0 : d0 - rh) : 0;
        float cv[CH], sv[CH];
        load8_or_4(cs + (int64_t)prow * rh + i0, cv);
        load8_or_4(sn + (int64_t)prow * rh + i0, sv);
#pragma unroll
        for (int e = 0; e < CH; ++e) {
          const float z = __shfl(x[e], src, 64);
          y[e] = x[e];
          if (rot_chunk) y[e] = d0 < rh ? x[e] * cv[e] - z * sv[e] : x[e] * cv[e] + z * sv[e];
        }
      }
#pragma unroll
      for (int e = 0; e < CH; ++e) x[e] = y[e];
    }
    if (row_ok) store8_or_4(static_cast<T*>(p.kc) + dst, x);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void copy_past_kernel(CopyPastParams p) {
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int total = p.lens[b] + 1;
  int rows = total - p.S, first = 0;
  if (p.win_cap > 0) {
    const WindowGeom g = window_geom(total, p.S, p.win_cap);
    first = g.drop;
    rows = min(g.held, p.past_seq) - g.drop;
  }
  rows = min(rows, min(p.past_seq - first, p.cap));
  if (rows <= 0) return;
  const int64_t n = (int64_t)rows * p.H;
  const T* sk = static_cast<const T*>(p.pk) + (((int64_t)b * p.kvN + kvh) * p.past_seq + first) * p.H;
  const T* sv = static_cast<const T*>(p.pv) + (((int64_t)b * p.kvN + kvh) * p.past_seq + first) * p.H;
  T* dk = static_cast<T*>(p.ck) + ((int64_t)b * p.kvN + kvh) * p.cap * p.H;
  T* dv = static_cast<T*>(p.cv) + ((int64_t)b * p.kvN + kvh) * p.cap * p.H;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    dk[i] = sk[i];
    dv[i] = sv[i];
  }
}

// Sliding-window eviction: rows [drop, held) of every (sample, kv head) slab
// of the keys and of the values (one workgroup each) move to
// [0, held - drop), as raw bytes in chunks of C (16, 8 or 4 bytes, the widest
// that divides a row: float rows, int8 code rows of H bytes, int4 rows of
// H / 2), in steps of whole rows (kShiftChunks chunks per thread).  A step
// loads all its rows before any is stored (barrier), so a step's stores may
// overwrite its own sources; the next step's sources lie above the rows
// stored so far (drop >= 1), so steps need no further ordering.
constexpr int kShiftThreads = 1024, kShiftChunks = 8;  // chunks per thread per step
template <typename C>
__global__ __launch_bounds__(kShiftThreads) void window_shift_kernel(WindowShiftParams p) {
  const int slab = blockIdx.x;           // (b, kvh)
  const int which = blockIdx.y;          // 0: keys, 1: values
  const int b = slab / p.kvN;
  const WindowGeom g = window_geom(p.lens[b] + 1, p.S, p.cap);
  const int keep = g.held - g.drop;
  if (g.drop <= 0 || keep <= 0) return;  // nothing moves (block-uniform)
  const int cpr = p.row_bytes / (int)sizeof(C);                 // chunks per row
  const int rows_step = kShiftThreads * kShiftChunks / cpr;     // whole rows per step
  {
    char* base = static_cast<char*>(which == 0 ? p.kc : p.vc) + (int64_t)slab * p.cap * p.row_bytes;
    for (int r0 = 0; r0 < keep; r0 += rows_step) {
      C v[kShiftChunks];
#pragma unroll
      for (int u = 0; u < kShiftChunks; ++u) {
        const int idx = threadIdx.x + kShiftThreads * u;
        const int r = r0 + idx / cpr, c = idx % cpr;
        if (r < keep && r < r0 + rows_step)
          v[u] = *reinterpret_cast<const C*>(base + ((int64_t)(r + g.drop) * cpr + c) * sizeof(C));
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kShiftChunks; ++u) {
        const int idx = threadIdx.x + kShiftThreads * u;
        const int r = r0 + idx / cpr, c = idx % cpr;
        if (r < keep && r < r0 + rows_step)
          *reinterpret_cast<C*>(base + ((int64_t)r * cpr + c) * sizeof(C)) = v[u];
      }
      __syncthreads();
    }
  }
}

}  // namespace

hipError_t launch_prep(DType dt, const PrepParams& p, hipStream_t s) {
  if (p.B * p.S == 0) return hipSuccess;
  const int ch = dt == DType::F16 ? 8 : 4;
  const int lpr = p.H / ch;  // lanes per row: a power of two (the norm sums by xor)
  const bool vec_ok = p.bits == 0 && p.kx == nullptr && !p.write_q && p.write_kv && p.H % ch == 0 && lpr <= 64 && (lpr & (lpr - 1)) == 0 &&
                      (p.cos == nullptr || p.interleaved || p.rot_half % ch == 0);
  if (vec_ok) {
    const int64_t rows = (int64_t)p.B * p.S * p.kvN;
    const int rows_per_wave = 64 / (p.H / ch);
    const int64_t waves = (rows + rows_per_wave - 1) / rows_per_wave;
    const int64_t blocks = std::min<int64_t>((waves + 3) / 4, 8192);
    if (dt == DType::F16)
      launch_kernel(prep_kv_kernel<f16>, dim3((int)blocks), dim3(kPrepThreads), 0, s, p);
    else
      launch_kernel(prep_kv_kernel<float>, dim3((int)blocks), dim3(kPrepThreads), 0, s, p);
    return hipGetLastError();
  }
  // few tokens (decode-sized calls): the heads of a token are spread over
  // several workgroups as well
  const int items = (p.write_q ? p.N : 0) + (p.write_kv ? 2 * p.kvN : 0);
  const int gy = (p.B * p.S < 1024) ? std::min((items + 3) / 4, 16) : 1;
  dim3 grid(p.B * p.S, std::max(gy, 1));
  if (dt == DType::F16)
    launch_kernel(prep_kernel<f16>, grid, dim3(kPrepThreads), 0, s, p);
  else
    launch_kernel(prep_kernel<float>, grid, dim3(kPrepThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_window_shift(const WindowShiftParams& p, hipStream_t s) {
  const int slabs = p.B * p.kvN;
  if (slabs == 0) return hipSuccess;
  if (p.row_bytes <= 0 || p.row_bytes % 4 != 0 || p.row_bytes > 1024) return hipErrorInvalidValue;
  // one workgroup per (slab, keys or values)
  const dim3 grid(slabs, 2);
  if (p.row_bytes % 16 == 0)
    launch_kernel(window_shift_kernel<uint4v>, grid, dim3(kShiftThreads), 0, s, p);
  else if (p.row_bytes % 8 == 0)
    launch_kernel(window_shift_kernel<uint2v>, grid, dim3(kShiftThreads), 0, s, p);
  else
    launch_kernel(window_shift_kernel<uint32_t>, grid, dim3(kShiftThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_copy_past(DType dt, const CopyPastParams& p, hipStream_t s) {
  if (p.B == 0 || p.kvN == 0) return hipSuccess;
  int64_t per = (int64_t)p.past_seq * p.H;
  int gx = (int)std::min<int64_t>((per + 255) / 256, 1024);
  if (gx < 1) gx = 1;
  dim3 grid(gx, p.kvN, p.B);
  if (dt == DType::F16)
    launch_kernel(copy_past_kernel<f16>, grid, dim3(256), 0, s, p);
  else if (dt == DType::Q8)
    launch_kernel(copy_past_kernel<int8_t>, grid, dim3(256), 0, s, p);
  else
    launch_kernel(copy_past_kernel<float>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvattn
