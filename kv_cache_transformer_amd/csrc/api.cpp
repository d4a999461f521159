// C ABI of the attention library: argument validation, launch planning and
// kernel launches.  Every check happens before the first launch, so a call
// that fails writes nothing.  The entry points never allocate, free or
// synchronise; all work goes to the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "kvattn.h"
#include "kvattn_internal.hpp"

using namespace kvattn;

kvattn::LaunchEvents& kvattn::launch_events() {
  thread_local LaunchEvents ev;
  return ev;
}

namespace {

thread_local std::string g_last_error;

// decode: waves per compute unit in the grid (two groups of four waves: two
// waves per SIMD)
constexpr int64_t kDecodeWavesPerCu = 8;
// decode: a wave streams at least this many keys when a unit is split
constexpr int64_t kDecodeMinKeysPerWave = 64;
// Every non-empty workspace starts with this many bytes of decode arrival
// counters (one int32 per split unit); no call writes anything else there,
// so one zero-filled workspace can serve calls of any operator and shape.
constexpr size_t kCounterBytes = KVATTN_COUNTER_BYTES;
constexpr int64_t kCounterSlots = kCounterBytes / sizeof(int32_t);

// measurement hook (kvattn_profile_events)
thread_local hipEvent_t g_prof_start = nullptr, g_prof_stop = nullptr;
thread_local int g_prof_kind = 0;

// decode grid fill target in waves per compute unit (kvattn_set_decode_split;
// 0 = kDecodeWavesPerCu)
thread_local int g_decode_waves_per_cu = 0;

// Run the launcher `f`; when `kind` is the one asked for, its first kernel
// records its own start and stop on the profiling events.
template <typename F>
hipError_t profiled(int kind, hipStream_t st, F&& f) {
  (void)st;
  const bool on = g_prof_kind == kind && g_prof_start != nullptr && g_prof_stop != nullptr;
  if (on) launch_events() = LaunchEvents{g_prof_start, g_prof_stop};
  const hipError_t e = f();
  launch_events() = LaunchEvents{};
  return e;
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return KVATTN_OK;
}

int64_t numel(const kvattn_tensor& t) {
  int64_t n = 1;
  for (int i = 0; i < t.rank && i < 4; ++i) n *= t.dims[i];
  return n;
}

// A tensor is present when it has data, or dims with no element (an empty
// tensor may come with a null pointer); absent slots are null with rank 0.
bool has(const kvattn_tensor& t) {
  return t.data != nullptr || (t.rank > 0 && t.rank <= 4 && numel(t) == 0);
}

std::string shape_str(const kvattn_tensor& t) {
  std::string s = "(";
  for (int i = 0; i < t.rank; ++i) {
    if (i) s += ", ";
    s += std::to_string((long long)t.dims[i]);
  }
  return s + ")";
}

// Check dtype, rank and dims (-1 = any) of a tensor.
int check(const kvattn_tensor& t, const char* name, int dtype, int rank,
          std::initializer_list<int64_t> dims) {
  if (t.dtype != dtype)
    return fail(KVATTN_ERR_INVALID_ARG, "%s: dtype %d, expected %d", name, t.dtype, dtype);
  if (t.rank != rank)
    return fail(KVATTN_ERR_INVALID_ARG, "%s: rank %d, expected %d", name, t.rank, rank);
  int i = 0;
  for (int64_t d : dims) {
    if (d >= 0 && t.dims[i] != d)
      return fail(KVATTN_ERR_INVALID_ARG, "%s: shape %s, dim %d expected %lld", name,
                  shape_str(t).c_str(), i, (long long)d);
    if (t.dims[i] < 0)
      return fail(KVATTN_ERR_INVALID_ARG, "%s: negative dim", name);
    ++i;
  }
  return KVATTN_OK;
}

#define CHECK(x)                       \
  do {                                 \
    int _rc = (x);                     \
    if (_rc != KVATTN_OK) return _rc;  \
  } while (0)

DType to_dtype(int dt) { return dt == KVATTN_DT_F16 ? DType::F16 : DType::F32; }
size_t elem_size(int dt) { return dt == KVATTN_DT_F16 ? 2 : 4; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int check_head_size(int H, const char* op) {
  if (H <= 0 || H % 8 != 0 || H > 256)
    return fail(KVATTN_ERR_UNSUPPORTED, "%s: head size %d (must be a multiple of 8, at most 256)", op, H);
  return KVATTN_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KVATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return KVATTN_OK;
}

// Compute units of the current device (cached per device; 256 when the
// query fails, e.g. without a GPU).
int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) return cache[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev >= 0 && dev < 64) cache[dev] = cus;
  return cus;
}

// Waves of the decode grid: enough to fill the device, no more than the
// units could use (a pair of waves streams >= 128 keys of a split unit), at
// least one pair per unit, a multiple of eight (workgroups of four pairs).
// kvattn_set_decode_split changes the fill target for the calling thread.
int64_t decode_waves(int64_t units, int64_t max_keys) {
  // more units than counter slots: one pair per unit (the grid is full
  // anyway; the kernel then splits nothing, see DecodeParams::split)
  if (units > kCounterSlots) return (2 * units + 7) / 8 * 8;
  const int64_t per_cu = g_decode_waves_per_cu > 0 ? g_decode_waves_per_cu : kDecodeWavesPerCu;
  const int64_t fill = per_cu * device_cu_count();
  const int64_t pair_keys = 2 * kDecodeMinKeysPerWave;
  const int64_t useful = 2 * (units + (units * std::max<int64_t>(max_keys, 0) + pair_keys - 1) / pair_keys);
  const int64_t w = std::max(2 * units, std::min(fill, useful));
  return (w + 7) / 8 * 8;
}

float resolve_scale(float scale, int H) {
  return scale == 0.f ? 1.f / std::sqrt((float)H) : scale;
}

// ===========================================================================
// GroupQueryAttention
// ===========================================================================
struct GqaPlan {
  int B, S, N, kvN, H, HP, cap, past_seq;
  int dt;
  bool has_past, shared, decode, q_transform;
  bool window_cache;  // sliding-window cache: fixed-size buffers evicting from the front
  int bits;           // quantised caches: 8 (int8) or 4 (packed nibbles); 0 = float caches
  bool k_pc, v_pc;    // per-channel scales
  int total;
  // decode
  int head_groups, hpw;
  int64_t waves;
  size_t ws_cnt, ws_q, ws_part, ws_total;  // workspace: counters first
  // a prompt's present cache in its own float type: the new rows in T for
  // the attention (keys, then values, each (B, kvN, S, H)) after the rest
  int cache_dt;
  bool own_cache_type;
  size_t ws_kv;
};

// Quantised-cache attributes and scales (GroupQueryAttention page,
// Attributes table: k_quant_type, v_quant_type, kv_cache_bit_width; Inputs
// table: k_scale, v_scale, and the requirement of float32 query/key/value
// and output; int4 caches are prompt-only).
int gqa_validate_quant(const gqa_attrs* a, const kvattn_tensor* in, int dt, GqaPlan& P) {
  const kvattn_tensor& ksc = in[GQA_IN_K_SCALE];
  const kvattn_tensor& vsc = in[GQA_IN_V_SCALE];
  P.bits = 0;
  P.k_pc = P.v_pc = false;
  if (a->kv_cache_bit_width == 0 && a->k_quant_type == 0 && a->v_quant_type == 0 && !has(ksc) && !has(vsc))
    return KVATTN_OK;
  if (a->kv_cache_bit_width != 8 && a->kv_cache_bit_width != 4)
    return fail(KVATTN_ERR_INVALID_ARG, "kv_cache_bit_width %d: quantised caches take 8 or 4", a->kv_cache_bit_width);
  for (int t : {a->k_quant_type, a->v_quant_type})
    if (t != GQA_QUANT_PER_TENSOR && t != GQA_QUANT_PER_CHANNEL)
      return fail(KVATTN_ERR_INVALID_ARG, "quantised caches need k_quant_type and v_quant_type PER_TENSOR (1) or PER_CHANNEL (2)");
  if (dt != KVATTN_DT_F32)
    return fail(KVATTN_ERR_INVALID_ARG, "quantised caches need float32 query, key, value and output");
  if (!has(ksc) || !has(vsc)) return fail(KVATTN_ERR_INVALID_ARG, "quantised caches need k_scale and v_scale");
  P.k_pc = a->k_quant_type == GQA_QUANT_PER_CHANNEL;
  P.v_pc = a->v_quant_type == GQA_QUANT_PER_CHANNEL;
  CHECK(check(ksc, "k_scale", KVATTN_DT_F32, 1, {P.k_pc ? (int64_t)P.kvN * P.H : 1}));
  CHECK(check(vsc, "v_scale", KVATTN_DT_F32, 1, {P.v_pc ? (int64_t)P.kvN * P.H : 1}));
  P.bits = a->kv_cache_bit_width;
  return KVATTN_OK;
}

int gqa_validate(const gqa_attrs* a, const kvattn_tensor* in, int n_in, int total,
                 const kvattn_tensor* out, int n_out, GqaPlan& P) {
  if (!a || !in || !out) return fail(KVATTN_ERR_INVALID_ARG, "gqa_attention: null argument");
  if (n_in != GQA_NUM_INPUTS || n_out != GQA_NUM_OUTPUTS)
    return fail(KVATTN_ERR_INVALID_ARG, "gqa_attention: expected %d inputs and %d outputs",
                GQA_NUM_INPUTS, GQA_NUM_OUTPUTS);
  const kvattn_tensor& q = in[GQA_IN_QUERY];
  if (!has(q)) return fail(KVATTN_ERR_INVALID_ARG, "query is required");
  if (q.dtype != KVATTN_DT_F16 && q.dtype != KVATTN_DT_F32)
    return fail(KVATTN_ERR_UNSUPPORTED, "query dtype %d: only float16 and float32", q.dtype);
  const int dt = q.dtype;
  CHECK(check(q, "query", dt, 3, {-1, -1, -1}));
  P.dt = dt;
  P.B = (int)q.dims[0];
  P.S = (int)q.dims[1];
  P.N = a->num_heads;
  P.kvN = a->kv_num_heads;
  if (P.N <= 0 || P.kvN <= 0 || P.N % P.kvN)
    return fail(KVATTN_ERR_INVALID_ARG, "num_heads %d / kv_num_heads %d: kv_num_heads must divide num_heads", P.N, P.kvN);
  if (q.dims[2] % P.N) return fail(KVATTN_ERR_INVALID_ARG, "query hidden %lld not divisible by num_heads", (long long)q.dims[2]);
  P.H = (int)(q.dims[2] / P.N);
  CHECK(check_head_size(P.H, "gqa_attention"));
  P.HP = padded_head(P.H);
  CHECK(gqa_validate_quant(a, in, dt, P));
  // cache element type and row width (elements): int8 rows of H, or H / 2
  // bytes of packed nibbles
  const int cdt = P.bits == 8 ? KVATTN_DT_I8 : (P.bits == 4 ? KVATTN_DT_U8 : dt);
  const int64_t Hc = P.bits == 4 ? P.H / 2 : P.H;
  if (a->sliding_window_cache != 0 && a->sliding_window_cache != 1)
    return fail(KVATTN_ERR_INVALID_ARG, "sliding_window_cache must be 0 or 1");
  P.window_cache = a->sliding_window_cache == 1;
  if (P.window_cache && (a->causal != 1 || a->local_window_size <= 0))
    return fail(KVATTN_ERR_INVALID_ARG, "sliding_window_cache needs causal = 1 and local_window_size > 0");
  if (a->causal != 0 && a->causal != 1) return fail(KVATTN_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (a->local_window_size < -1) return fail(KVATTN_ERR_INVALID_ARG, "local_window_size must be >= -1");
  if (!a->causal && a->local_window_size != -1)
    return fail(KVATTN_ERR_INVALID_ARG, "causal = 0 requires local_window_size = -1");
  if (!(a->softcap >= 0.f)) return fail(KVATTN_ERR_INVALID_ARG, "softcap must be >= 0");
  if (!std::isfinite(a->scale)) return fail(KVATTN_ERR_INVALID_ARG, "scale must be finite");

  const kvattn_tensor& k = in[GQA_IN_KEY];
  const kvattn_tensor& v = in[GQA_IN_VALUE];
  if (!has(k) || !has(v)) return fail(KVATTN_ERR_UNSUPPORTED, "packed QKV (no key/value) is not implemented");
  CHECK(check(k, "key", dt, 3, {P.B, -1, (int64_t)P.kvN * P.H}));
  CHECK(check(v, "value", dt, 3, {P.B, k.dims[1], (int64_t)P.kvN * P.H}));
  if (k.dims[1] != P.S) return fail(KVATTN_ERR_UNSUPPORTED, "kv_sequence_length %lld != sequence_length %d", (long long)k.dims[1], P.S);

  const kvattn_tensor& pk = in[GQA_IN_PAST_KEY];
  const kvattn_tensor& pv = in[GQA_IN_PAST_VALUE];
  if (has(pk) != has(pv)) return fail(KVATTN_ERR_INVALID_ARG, "past_key and past_value go together");
  P.has_past = has(pk);
  if (P.has_past) {
    if (!a->causal) return fail(KVATTN_ERR_UNSUPPORTED, "bidirectional attention takes no past cache");
    CHECK(check(pk, "past_key", cdt, 4, {P.B, P.kvN, -1, Hc}));
    CHECK(check(pv, "past_value", cdt, 4, {P.B, P.kvN, pk.dims[2], Hc}));
    P.past_seq = (int)pk.dims[2];
  } else {
    P.past_seq = 0;
  }
  const kvattn_tensor& sl = in[GQA_IN_SEQLENS_K];
  if (!has(sl)) return fail(KVATTN_ERR_INVALID_ARG, "seqlens_k is required");
  CHECK(check(sl, "seqlens_k", KVATTN_DT_I32, 1, {P.B}));
  if (total < 1) return fail(KVATTN_ERR_INVALID_ARG, "total_sequence_length must be >= 1");
  P.total = total;

  const kvattn_tensor& o = out[GQA_OUT_OUTPUT];
  const kvattn_tensor& ck = out[GQA_OUT_PRESENT_KEY];
  const kvattn_tensor& cv = out[GQA_OUT_PRESENT_VALUE];
  if (!has(o) || !has(ck) || !has(cv)) return fail(KVATTN_ERR_INVALID_ARG, "output, present_key and present_value are required");
  CHECK(check(o, "output", dt, 3, {P.B, P.S, (int64_t)P.N * P.H}));
  // without a past the float cache may be float16 or float32 whatever T is
  // (GroupQueryAttention page, Description); a past fixes it to T
  P.cache_dt = cdt;
  if (P.bits == 0 && !P.has_past && (ck.dtype == KVATTN_DT_F16 || ck.dtype == KVATTN_DT_F32))
    P.cache_dt = ck.dtype;
  P.own_cache_type = P.cache_dt != cdt;
  CHECK(check(ck, "present_key", P.cache_dt, 4, {P.B, P.kvN, -1, Hc}));
  CHECK(check(cv, "present_value", P.cache_dt, 4, {P.B, P.kvN, ck.dims[2], Hc}));
  P.cap = (int)ck.dims[2];
  P.shared = P.has_past && ck.data == pk.data;
  if (P.has_past && ((cv.data == pv.data) != P.shared))
    return fail(KVATTN_ERR_INVALID_ARG, "present_key and present_value must both share the past buffers or neither");
  if (P.shared && ck.dims[2] != pk.dims[2])
    return fail(KVATTN_ERR_INVALID_ARG, "a shared present buffer must have the past buffer's dims");
  if (P.bits == 4 && P.has_past && P.S == 1 && P.H % (P.HP / 8) != 0)
    return fail(KVATTN_ERR_UNSUPPORTED, "int4 decode: head size %d must be a multiple of %d", P.H, P.HP / 8);
  if (P.window_cache) {
    if (!P.has_past)
      return fail(KVATTN_ERR_INVALID_ARG, "sliding_window_cache needs a past cache");
    // separate buffers: the past holds the window before the call, at most
    // min(total - S, capacity) rows
    if (!P.shared && P.past_seq < std::min<int64_t>(std::max<int64_t>(total - P.S, 0), P.cap))
      return fail(KVATTN_ERR_INVALID_ARG, "sliding_window_cache: past sequence axis %d cannot hold the window (%lld rows)",
                  P.past_seq, (long long)std::min<int64_t>(total - P.S, P.cap));
    if (P.cap < a->local_window_size + P.S)
      return fail(KVATTN_ERR_INVALID_ARG, "sliding_window_cache: capacity %d < local_window_size + sequence_length (%d)",
                  P.cap, a->local_window_size + P.S);
    if (has(in[GQA_IN_ATTENTION_BIAS]))
      return fail(KVATTN_ERR_UNSUPPORTED, "sliding_window_cache with attention_bias is not implemented");
  } else if (P.has_past && P.cap < total) {
    return fail(KVATTN_ERR_INVALID_ARG, "present sequence axis %d cannot hold total_sequence_length %d", P.cap, total);
  }
  if (!P.has_past && P.cap < P.S)
    return fail(KVATTN_ERR_INVALID_ARG, "present sequence axis %d < sequence_length %d", P.cap, P.S);

  const kvattn_tensor& cs = in[GQA_IN_COS_CACHE];
  const kvattn_tensor& sn = in[GQA_IN_SIN_CACHE];
  if (a->do_rotary) {
    if (!has(cs) || !has(sn)) return fail(KVATTN_ERR_INVALID_ARG, "do_rotary needs cos_cache and sin_cache");
    CHECK(check(cs, "cos_cache", dt, 2, {-1, P.H / 2}));
    CHECK(check(sn, "sin_cache", dt, 2, {cs.dims[0], P.H / 2}));
    const int need = P.has_past ? total : P.S;
    if (cs.dims[0] < need)
      return fail(KVATTN_ERR_INVALID_ARG, "cos_cache has %lld rows, positions up to %d are used", (long long)cs.dims[0], need - 1);
  }
  const kvattn_tensor& bias = in[GQA_IN_ATTENTION_BIAS];
  if (has(bias)) {
    CHECK(check(bias, "attention_bias", dt, 4, {-1, -1, P.S, a->causal ? total : P.S}));
    if (bias.dims[0] != 1 && bias.dims[0] != P.B) return fail(KVATTN_ERR_INVALID_ARG, "attention_bias dim 0 must be 1 or batch");
    if (bias.dims[1] != 1 && bias.dims[1] != P.N) return fail(KVATTN_ERR_INVALID_ARG, "attention_bias dim 1 must be 1 or num_heads");
  }
  if (has(in[GQA_IN_HEAD_SINK])) CHECK(check(in[GQA_IN_HEAD_SINK], "head_sink", dt, 1, {P.N}));
  const bool qn = has(in[GQA_IN_Q_NORM_WEIGHT]), kn = has(in[GQA_IN_K_NORM_WEIGHT]);
  if (qn != kn) return fail(KVATTN_ERR_INVALID_ARG, "q_norm_weight and k_norm_weight must be given together");
  if (qn) {
    CHECK(check(in[GQA_IN_Q_NORM_WEIGHT], "q_norm_weight", dt, 1, {P.H}));
    CHECK(check(in[GQA_IN_K_NORM_WEIGHT], "k_norm_weight", dt, 1, {P.H}));
  }

  P.decode = P.has_past && P.S == 1;
  P.q_transform = qn || a->do_rotary;
  size_t esz = elem_size(dt);
  P.ws_cnt = 0;
  P.ws_q = 0;
  P.ws_part = 0;
  if (P.decode) {
    const int g = P.N / P.kvN;
    P.head_groups = (g + 15) / 16;
    P.hpw = std::min(16, g);
    const int64_t units = (int64_t)P.B * P.kvN * P.head_groups;
    P.waves = decode_waves(units, std::min<int64_t>(total, P.cap));
    if (P.waves > (int64_t)1 << 30) return fail(KVATTN_ERR_INVALID_ARG, "decode: too many (sample, head) units");
    P.ws_part = align256((size_t)(P.waves / 2) * P.hpw * (P.HP + 4) * sizeof(float));
  }
  P.ws_kv = P.own_cache_type ? align256(2 * (size_t)P.B * P.kvN * P.S * P.H * esz) : 0;
  // every non-empty workspace starts with the arrival counters, which no
  // other use may touch
  const size_t body = P.ws_q + P.ws_part + P.ws_kv;
  P.ws_cnt = body ? kCounterBytes : 0;
  P.ws_total = P.ws_cnt + body;
  return KVATTN_OK;
}

int gqa_run(const gqa_attrs* a, const kvattn_tensor* in, const kvattn_tensor* out,
            const GqaPlan& P, void* ws, hipStream_t st) {
  const DType dt = to_dtype(P.dt);
  const kvattn_tensor& ck = out[GQA_OUT_PRESENT_KEY];
  const kvattn_tensor& cv = out[GQA_OUT_PRESENT_VALUE];
  const float scale = resolve_scale(a->scale, P.H);
  char* wsb = static_cast<char*>(ws);

  if (P.has_past && !P.shared) {
    CopyPastParams c{};
    c.pk = in[GQA_IN_PAST_KEY].data;
    c.pv = in[GQA_IN_PAST_VALUE].data;
    c.ck = ck.data;
    c.cv = cv.data;
    c.lens = static_cast<const int32_t*>(in[GQA_IN_SEQLENS_K].data);
    // quantised caches copy bytes: H codes (int8) or H / 2 bytes (int4) per row
    c.B = P.B; c.kvN = P.kvN; c.H = P.bits == 4 ? P.H / 2 : P.H; c.S = P.S; c.past_seq = P.past_seq; c.cap = P.cap;
    // sliding-window cache over separate buffers: the copy moves the rows
    // that survive the eviction to the front (the shift of the shared case)
    c.win_cap = P.window_cache ? P.cap : 0;
    CHECK(hip_status(launch_copy_past(P.bits != 0 ? DType::Q8 : dt, c, st), "copy_past launch"));
  }

  if (P.window_cache && P.shared) {
    WindowShiftParams w{};
    w.kc = ck.data;
    w.vc = cv.data;
    w.lens = static_cast<const int32_t*>(in[GQA_IN_SEQLENS_K].data);
    w.B = P.B; w.kvN = P.kvN; w.S = P.S; w.cap = P.cap;
    // quantised caches move code rows: H bytes (int8) or H / 2 (int4)
    w.row_bytes = P.bits == 8 ? P.H : (P.bits == 4 ? P.H / 2 : P.H * (int)elem_size(P.dt));
    CHECK(hip_status(profiled(KVATTN_PROFILE_SHIFT, st, [&] { return launch_window_shift(w, st); }),
                     "window shift launch"));
  }

  const kvattn_tensor& bias = in[GQA_IN_ATTENTION_BIAS];
  if (P.decode) {
    DecodeParams d{};
    d.q = in[GQA_IN_QUERY].data;
    d.k_new = in[GQA_IN_KEY].data;
    d.v_new = in[GQA_IN_VALUE].data;
    d.kc = ck.data;
    d.vc = cv.data;
    d.q_norm = in[GQA_IN_Q_NORM_WEIGHT].data;
    d.k_norm = in[GQA_IN_K_NORM_WEIGHT].data;
    d.eps = a->qk_norm_epsilon;
    if (a->do_rotary) {
      d.cos = in[GQA_IN_COS_CACHE].data;
      d.sin = in[GQA_IN_SIN_CACHE].data;
      d.rot_rows = (int)in[GQA_IN_COS_CACHE].dims[0];
    }
    if (has(bias)) {
      d.bias = bias.data;
      d.bias_cols = (int)bias.dims[3];
      d.bias_sb = bias.dims[0] > 1 ? bias.dims[1] * bias.dims[3] : 0;
      d.bias_sh = bias.dims[1] > 1 ? bias.dims[3] : 0;
    }
    d.sink = in[GQA_IN_HEAD_SINK].data;
    d.smooth = a->smooth_softmax == 1;
    d.lens = static_cast<const int32_t*>(in[GQA_IN_SEQLENS_K].data);
    d.len_mode = 0;
    d.window = a->local_window_size;
    d.win_cap = P.window_cache ? P.cap : 0;
    d.out = out[GQA_OUT_OUTPUT].data;
    d.counters = reinterpret_cast<int*>(wsb);
    d.part = reinterpret_cast<float*>(wsb + P.ws_cnt + P.ws_q);
    d.B = P.B; d.N = P.N; d.kvN = P.kvN; d.H = P.H; d.cap = P.cap;
    d.scale = scale;
    d.softcap = a->softcap;
    d.head_groups = P.head_groups; d.hpw = P.hpw; d.waves = (int)P.waves;
    d.split = (int64_t)d.B * d.kvN * d.head_groups <= kCounterSlots;
    d.k_scale = static_cast<const float*>(in[GQA_IN_K_SCALE].data);
    d.v_scale = static_cast<const float*>(in[GQA_IN_V_SCALE].data);
    d.k_scale_pc = P.k_pc;
    d.v_scale_pc = P.v_pc;
    const DType ddt = P.bits == 8 ? DType::Q8 : (P.bits == 4 ? DType::Q4 : dt);
    CHECK(hip_status(profiled(KVATTN_PROFILE_DECODE, st, [&] { return launch_decode(ddt, P.HP, d, st); }),
                     "decode launch"));
    return ok();
  }

  // prefill: prep (k/v into the cache, transformed queries), then flash
  PrepParams pp{};
  pp.q = in[GQA_IN_QUERY].data;
  pp.k = in[GQA_IN_KEY].data;
  pp.v = in[GQA_IN_VALUE].data;
  pp.q_stride = (int64_t)P.N * P.H;
  pp.k_stride = pp.v_stride = (int64_t)P.kvN * P.H;
  pp.q_out = nullptr;  // the flash kernel prepares the queries as it loads them
  pp.kc = ck.data;
  pp.vc = cv.data;
  pp.q_norm = in[GQA_IN_Q_NORM_WEIGHT].data;
  pp.k_norm = in[GQA_IN_K_NORM_WEIGHT].data;
  pp.eps = a->qk_norm_epsilon;
  if (a->do_rotary) {
    pp.cos = in[GQA_IN_COS_CACHE].data;
    pp.sin = in[GQA_IN_SIN_CACHE].data;
    pp.rot_half = P.H / 2;
    pp.rot_rows = (int)in[GQA_IN_COS_CACHE].dims[0];
  }
  pp.lens = static_cast<const int32_t*>(in[GQA_IN_SEQLENS_K].data);
  pp.pos_mode = P.has_past ? 1 : 0;
  pp.B = P.B; pp.S = P.S; pp.N = P.N; pp.kvN = P.kvN; pp.H = P.H; pp.cap = P.cap;
  pp.write_q = 0;
  pp.write_kv = 1;
  pp.win_cap = P.window_cache ? P.cap : 0;
  // quantised prompt: codes into the present caches, which the attention
  // reads and widens itself (no float copy)
  // a present cache of another float type: the rows in T go to the
  // workspace, which the attention reads, and to the cache in its type
  void* att_k = ck.data;
  void* att_v = cv.data;
  int att_rows = P.cap;
  if (P.own_cache_type) {
    const size_t half = (size_t)P.B * P.kvN * P.S * P.H * elem_size(P.dt);
    att_k = wsb + P.ws_cnt + P.ws_q + P.ws_part;
    att_v = static_cast<char*>(att_k) + half;
    att_rows = P.S;
    pp.kc = att_k;
    pp.vc = att_v;
    pp.cap = P.S;
    pp.kx = ck.data;
    pp.vx = cv.data;
    pp.xcap = P.cap;
    pp.x_f32 = P.cache_dt == KVATTN_DT_F32;
  }
  if (P.bits != 0) {
    pp.bits = P.bits;
    pp.kq = ck.data;
    pp.vq = cv.data;
    pp.qcap = P.cap;
    pp.kc = nullptr;
    pp.vc = nullptr;
    pp.k_scale = static_cast<const float*>(in[GQA_IN_K_SCALE].data);
    pp.v_scale = static_cast<const float*>(in[GQA_IN_V_SCALE].data);
    pp.k_scale_pc = P.k_pc;
    pp.v_scale_pc = P.v_pc;
  }
  CHECK(hip_status(profiled(KVATTN_PROFILE_PREP, st, [&] { return launch_prep(dt, pp, st); }),
                   "prep launch"));

  FlashParams f{};
  f.q = in[GQA_IN_QUERY].data;
  f.q_norm = pp.q_norm;
  f.eps = a->qk_norm_epsilon;
  f.cos = pp.cos;
  f.sin = pp.sin;
  f.rot_half = pp.rot_half;
  f.rot_rows = pp.rot_rows;
  f.interleaved = 0;
  f.q_s = (int64_t)P.N * P.H;
  f.q_b = f.q_s * P.S;
  f.q_h = P.H;
  f.kc = att_k;
  f.vc = att_v;
  f.k_j = P.H;
  f.k_h = (int64_t)att_rows * P.H;
  f.k_b = f.k_h * P.kvN;
  if (P.bits != 0) {
    f.qbits = P.bits;
    f.qk_scale = static_cast<const float*>(in[GQA_IN_K_SCALE].data);
    f.qv_scale = static_cast<const float*>(in[GQA_IN_V_SCALE].data);
    f.qk_pc = P.k_pc;
    f.qv_pc = P.v_pc;
  }
  f.out = out[GQA_OUT_OUTPUT].data;
  f.o_s = (int64_t)P.N * P.H;
  f.o_b = f.o_s * P.S;
  f.o_h = P.H;
  if (has(bias)) {
    f.bias = bias.data;
    const int64_t cols = bias.dims[3];
    f.bias_ss = cols;
    f.bias_sh = bias.dims[1] > 1 ? P.S * cols : 0;
    f.bias_sb = bias.dims[0] > 1 ? bias.dims[1] * P.S * cols : 0;
    f.bias_cols = (int)cols;
  }
  f.sink = in[GQA_IN_HEAD_SINK].data;
  f.smooth = a->smooth_softmax == 1;
  f.lens = static_cast<const int32_t*>(in[GQA_IN_SEQLENS_K].data);
  f.has_past = P.has_past;
  f.win_cap = P.window_cache ? P.cap : 0;
  f.causal = a->causal;
  f.window = a->local_window_size;
  f.kv_rows = att_rows;
  f.B = P.B; f.S = P.S; f.N = P.N; f.kvN = P.kvN; f.H = P.H;
  f.scale = scale;
  f.softcap = a->softcap;
  const int g = P.N / P.kvN;
  const int hw = (g % 4 == 0) ? 4 : (g % 2 == 0 ? 2 : 1);
  f.heads_per_wg = hw;
  f.rows_per_wg = 128 / hw;  // four waves of 32 rows
  f.mode = kDense;
  const int gx = (P.S + f.rows_per_wg - 1) / f.rows_per_wg;
  CHECK(hip_status(profiled(KVATTN_PROFILE_FLASH, st,
                            [&] { return launch_flash(dt, P.HP, f, gx, P.kvN * (g / hw), P.B, st); }),
                   "flash launch"));
  return ok();
}

// ===========================================================================
// DecoderMaskedMultiHeadAttention
// ===========================================================================
struct DmmhaPlan {
  int B, N, H, HP, dt, cap, kv_len;
  bool self;
  int64_t waves;
  size_t ws_cnt, ws_total;  // workspace: arrival counters, then partials
};

int dmmha_validate(const dmmha_attrs* a, const kvattn_tensor* in, int n_in,
                   const kvattn_tensor* out, int n_out, DmmhaPlan& P) {
  if (!a || !in || !out) return fail(KVATTN_ERR_INVALID_ARG, "decode_mha: null argument");
  if (n_in != DMMHA_NUM_INPUTS || n_out != DMMHA_NUM_OUTPUTS)
    return fail(KVATTN_ERR_INVALID_ARG, "decode_mha: expected %d inputs and %d outputs", DMMHA_NUM_INPUTS, DMMHA_NUM_OUTPUTS);
  const kvattn_tensor& q = in[DMMHA_IN_QUERY];
  if (!has(q)) return fail(KVATTN_ERR_INVALID_ARG, "query is required");
  if (q.dtype != KVATTN_DT_F16 && q.dtype != KVATTN_DT_F32)
    return fail(KVATTN_ERR_UNSUPPORTED, "query dtype %d: only float16 and float32", q.dtype);
  const int dt = q.dtype;
  P.dt = dt;
  CHECK(check(q, "query", dt, 3, {-1, 1, -1}));
  P.B = (int)q.dims[0];
  P.N = a->num_heads;
  if (P.N <= 0 || q.dims[2] % P.N) return fail(KVATTN_ERR_INVALID_ARG, "num_heads %d must divide the query hidden size", P.N);
  P.H = (int)(q.dims[2] / P.N);
  CHECK(check_head_size(P.H, "decode_mha"));
  P.HP = padded_head(P.H);
  if (!std::isfinite(a->scale) || !std::isfinite(a->mask_filter_value))
    return fail(KVATTN_ERR_INVALID_ARG, "scale and mask_filter_value must be finite");
  const kvattn_tensor& k = in[DMMHA_IN_KEY];
  const kvattn_tensor& v = in[DMMHA_IN_VALUE];
  if (!has(k) || !has(v)) return fail(KVATTN_ERR_INVALID_ARG, "key and value are required");
  const kvattn_tensor& pk = in[DMMHA_IN_PAST_KEY];
  const kvattn_tensor& pv = in[DMMHA_IN_PAST_VALUE];
  if (has(pk) != has(pv)) return fail(KVATTN_ERR_INVALID_ARG, "past_key and past_value go together");
  P.self = has(pk);
  const kvattn_tensor& o = out[DMMHA_OUT_OUTPUT];
  if (!has(o)) return fail(KVATTN_ERR_INVALID_ARG, "output is required");
  CHECK(check(o, "output", dt, 3, {P.B, 1, (int64_t)P.N * P.H}));
  const kvattn_tensor& qk = out[DMMHA_OUT_QK];
  if (P.self) {
    if (a->past_present_share_buffer != 1)
      return fail(KVATTN_ERR_INVALID_ARG, "self attention requires past_present_share_buffer = 1");
    CHECK(check(k, "key", dt, 3, {P.B, 1, (int64_t)P.N * P.H}));
    CHECK(check(v, "value", dt, 3, {P.B, 1, (int64_t)P.N * P.H}));
    CHECK(check(pk, "past_key", dt, 4, {P.B, P.N, -1, P.H}));
    CHECK(check(pv, "past_value", dt, 4, {P.B, P.N, pk.dims[2], P.H}));
    P.cap = (int)pk.dims[2];
    if (P.cap < 1) return fail(KVATTN_ERR_INVALID_ARG, "past_key capacity must be >= 1");
    const kvattn_tensor& psl = in[DMMHA_IN_PAST_SEQUENCE_LENGTH];
    if (!has(psl)) return fail(KVATTN_ERR_INVALID_ARG, "self attention needs past_sequence_length");
    if (psl.dtype != KVATTN_DT_I32 || numel(psl) != 1)
      return fail(KVATTN_ERR_INVALID_ARG, "past_sequence_length must hold one int32");
    const kvattn_tensor& ck = out[DMMHA_OUT_PRESENT_KEY];
    const kvattn_tensor& cv = out[DMMHA_OUT_PRESENT_VALUE];
    if ((has(ck) && ck.data != pk.data) || (has(cv) && cv.data != pv.data))
      return fail(KVATTN_ERR_INVALID_ARG, "present_key/present_value must be the past buffers (shared) or absent");
    if (a->output_qk || has(qk))
      return fail(KVATTN_ERR_INVALID_ARG, "qk is produced for cross attention only");
    P.kv_len = P.cap;
  } else {
    if (a->past_present_share_buffer != 0)
      return fail(KVATTN_ERR_INVALID_ARG, "cross attention has no cache: past_present_share_buffer must be 0");
    CHECK(check(k, "key", dt, 4, {P.B, P.N, -1, P.H}));
    CHECK(check(v, "value", dt, 4, {P.B, P.N, k.dims[2], P.H}));
    P.kv_len = (int)k.dims[2];
    P.cap = P.kv_len;
    if (P.kv_len < 1) return fail(KVATTN_ERR_INVALID_ARG, "key must hold at least one position");
    if (has(in[DMMHA_IN_ATTENTION_BIAS]))
      return fail(KVATTN_ERR_INVALID_ARG, "attention_bias is for self attention only");
    if (has(out[DMMHA_OUT_PRESENT_KEY]) || has(out[DMMHA_OUT_PRESENT_VALUE]))
      return fail(KVATTN_ERR_INVALID_ARG, "cross attention has no present cache");
    if ((a->output_qk != 0) != has(qk))
      return fail(KVATTN_ERR_INVALID_ARG, "output_qk must agree with the presence of the qk output");
    // qk has its own type, float32 or float16, whatever T is
    if (has(qk)) CHECK(check(qk, "qk", qk.dtype == KVATTN_DT_F32 ? KVATTN_DT_F32 : KVATTN_DT_F16, 4,
                             {P.B, P.N, 1, P.kv_len}));
  }
  const kvattn_tensor& m = in[DMMHA_IN_MASK_INDEX];
  if (has(m)) {
    CHECK(check(m, "mask_index", KVATTN_DT_I32, 2, {P.B, -1}));
    if (!P.self && m.dims[1] != P.kv_len) return fail(KVATTN_ERR_INVALID_ARG, "mask_index must be (batch, kv_sequence_length)");
  }
  const kvattn_tensor& bias = in[DMMHA_IN_ATTENTION_BIAS];
  if (has(bias)) {
    CHECK(check(bias, "attention_bias", dt, 4, {-1, -1, 1, -1}));
    if (bias.dims[0] != 1 && bias.dims[0] != P.B) return fail(KVATTN_ERR_INVALID_ARG, "attention_bias dim 0 must be 1 or batch");
    if (bias.dims[1] != 1 && bias.dims[1] != P.N) return fail(KVATTN_ERR_INVALID_ARG, "attention_bias dim 1 must be 1 or num_heads");
  }
  const int64_t units = (int64_t)P.B * P.N;
  P.waves = decode_waves(units, P.kv_len);
  if (P.waves > (int64_t)1 << 30) return fail(KVATTN_ERR_INVALID_ARG, "decode_mha: too many (sample, head) units");
  P.ws_cnt = kCounterBytes;
  P.ws_total = P.ws_cnt + align256((size_t)(P.waves / 2) * (P.HP + 4) * sizeof(float));
  return KVATTN_OK;
}

int dmmha_run(const dmmha_attrs* a, const kvattn_tensor* in, const kvattn_tensor* out,
              const DmmhaPlan& P, void* ws, hipStream_t st) {
  DecodeParams d{};
  d.q = in[DMMHA_IN_QUERY].data;
  if (P.self) {
    d.k_new = in[DMMHA_IN_KEY].data;
    d.v_new = in[DMMHA_IN_VALUE].data;
    d.kc = in[DMMHA_IN_PAST_KEY].data;
    d.vc = in[DMMHA_IN_PAST_VALUE].data;
    d.lens = static_cast<const int32_t*>(in[DMMHA_IN_PAST_SEQUENCE_LENGTH].data);
    d.len_mode = 1;
  } else {
    d.kc = in[DMMHA_IN_KEY].data;
    d.vc = in[DMMHA_IN_VALUE].data;
    d.len_mode = 2;
    d.host_n = P.kv_len;
    d.qk = out[DMMHA_OUT_QK].data;
    d.qk_f32 = out[DMMHA_OUT_QK].dtype == KVATTN_DT_F32;
  }
  const kvattn_tensor& bias = in[DMMHA_IN_ATTENTION_BIAS];
  if (has(bias)) {
    d.bias = bias.data;
    d.bias_cols = (int)bias.dims[3];
    d.bias_sb = bias.dims[0] > 1 ? bias.dims[1] * bias.dims[3] : 0;
    d.bias_sh = bias.dims[1] > 1 ? bias.dims[3] : 0;
  }
  const kvattn_tensor& m = in[DMMHA_IN_MASK_INDEX];
  if (has(m)) {
    d.mask = static_cast<const int32_t*>(m.data);
    d.mask_cols = (int)m.dims[1];
  }
  d.mask_filter = a->mask_filter_value;
  d.window = -1;
  d.out = out[DMMHA_OUT_OUTPUT].data;
  d.counters = static_cast<int*>(ws);
  d.part = reinterpret_cast<float*>(static_cast<char*>(ws) + P.ws_cnt);
  d.B = P.B; d.N = P.N; d.kvN = P.N; d.H = P.H; d.cap = P.cap;
  d.scale = resolve_scale(a->scale, P.H);
  d.head_groups = 1; d.hpw = 1; d.waves = (int)P.waves;
  d.split = (int64_t)d.B * d.kvN * d.head_groups <= kCounterSlots;
  CHECK(hip_status(profiled(KVATTN_PROFILE_DECODE, st,
                            [&] { return launch_decode(to_dtype(P.dt), P.HP, d, st); }),
                   "decode launch"));
  return ok();
}

// ===========================================================================
// SparseAttention
// ===========================================================================
struct SparsePlan {
  int B, S, N, kvN, H, HP, dt, cap, L, max_blocks, max_nnz, rot_half, bs;
  bool packed_qkv, rotary, generation;
  bool decode;      // one new token: split-key decode over the CSR blocks
  int64_t waves;
  size_t ws_cnt, ws_q, ws_part, ws_total;  // workspace: counters first
};

// most CSR blocks per row the decode route takes (its block table sits in LDS)
constexpr int kSparseDecodeMaxBlocks = 4096;

int sparse_validate(const sparse_attrs* a, const kvattn_tensor* in, int n_in, int total,
                    const kvattn_tensor* out, int n_out, SparsePlan& P) {
  if (!a || !in || !out) return fail(KVATTN_ERR_INVALID_ARG, "sparse_attention: null argument");
  if (n_in != SPARSE_NUM_INPUTS || n_out != SPARSE_NUM_OUTPUTS)
    return fail(KVATTN_ERR_INVALID_ARG, "sparse_attention: expected %d inputs and %d outputs", SPARSE_NUM_INPUTS, SPARSE_NUM_OUTPUTS);
  const kvattn_tensor& q = in[SPARSE_IN_QUERY];
  if (!has(q)) return fail(KVATTN_ERR_INVALID_ARG, "query is required");
  if (q.dtype != KVATTN_DT_F16 && q.dtype != KVATTN_DT_F32)
    return fail(KVATTN_ERR_UNSUPPORTED, "query dtype %d: only float16 and float32", q.dtype);
  const int dt = q.dtype;
  P.dt = dt;
  CHECK(check(q, "query", dt, 3, {-1, -1, -1}));
  P.B = (int)q.dims[0];
  P.S = (int)q.dims[1];
  P.N = a->num_heads;
  P.kvN = a->kv_num_heads;
  if (P.N <= 0 || P.kvN <= 0 || P.N % P.kvN)
    return fail(KVATTN_ERR_INVALID_ARG, "kv_num_heads must divide num_heads");
  const kvattn_tensor& k = in[SPARSE_IN_KEY];
  const kvattn_tensor& v = in[SPARSE_IN_VALUE];
  if (has(k) != has(v)) return fail(KVATTN_ERR_INVALID_ARG, "key and value go together");
  P.packed_qkv = !has(k);
  const int64_t width = q.dims[2];
  const int64_t heads = P.packed_qkv ? (P.N + 2 * P.kvN) : P.N;
  if (width % heads) return fail(KVATTN_ERR_INVALID_ARG, "query width %lld not divisible by %lld heads", (long long)width, (long long)heads);
  P.H = (int)(width / heads);
  if (P.H <= 0 || P.H % 8) return fail(KVATTN_ERR_INVALID_ARG, "head size %d must be a non-zero multiple of 8", P.H);
  CHECK(check_head_size(P.H, "sparse_attention"));
  P.HP = padded_head(P.H);
  if (!P.packed_qkv) {
    CHECK(check(k, "key", dt, 3, {P.B, P.S, (int64_t)P.kvN * P.H}));
    CHECK(check(v, "value", dt, 3, {P.B, P.S, (int64_t)P.kvN * P.H}));
  }
  const kvattn_tensor& pk = in[SPARSE_IN_PAST_KEY];
  const kvattn_tensor& pv = in[SPARSE_IN_PAST_VALUE];
  if (!has(pk) || !has(pv)) return fail(KVATTN_ERR_INVALID_ARG, "past_key and past_value are required");
  CHECK(check(pk, "past_key", dt, 4, {P.B, P.kvN, -1, P.H}));
  CHECK(check(pv, "past_value", dt, 4, {P.B, P.kvN, pk.dims[2], P.H}));
  P.cap = (int)pk.dims[2];
  const int bs = a->sparse_block_size;
  if (bs != 16 && bs != 32 && bs != 64 && bs != 128)
    return fail(KVATTN_ERR_INVALID_ARG, "sparse_block_size %d must be 16, 32, 64 or 128", bs);
  P.bs = bs;
  const kvattn_tensor& rp = in[SPARSE_IN_BLOCK_ROW_INDICES];
  const kvattn_tensor& cols = in[SPARSE_IN_BLOCK_COL_INDICES];
  if (!has(rp) || !has(cols)) return fail(KVATTN_ERR_INVALID_ARG, "block_row_indices and block_col_indices are required");
  CHECK(check(rp, "block_row_indices", KVATTN_DT_I32, 2, {-1, -1}));
  CHECK(check(cols, "block_col_indices", KVATTN_DT_I32, 2, {rp.dims[0], -1}));
  P.L = (int)rp.dims[0];
  P.max_blocks = (int)rp.dims[1] - 1;
  P.max_nnz = (int)cols.dims[1];
  if (P.L < 1 || P.max_blocks < 1) return fail(KVATTN_ERR_INVALID_ARG, "block_row_indices must be (num_layout >= 1, max_blocks + 1 >= 2)");
  const kvattn_tensor& kt = in[SPARSE_IN_KEY_TOTAL_SEQUENCE_LENGTHS];
  if (!has(kt)) return fail(KVATTN_ERR_INVALID_ARG, "key_total_sequence_lengths is required");
  CHECK(check(kt, "key_total_sequence_lengths", KVATTN_DT_I32, 1, {P.B}));
  if (total < 1) return fail(KVATTN_ERR_INVALID_ARG, "total_sequence_length must be >= 1");
  if (total > P.cap) return fail(KVATTN_ERR_INVALID_ARG, "total_sequence_length %d exceeds the cache capacity %d", total, P.cap);
  if ((int64_t)total > (int64_t)P.max_blocks * bs)
    return fail(KVATTN_ERR_INVALID_ARG, "total_sequence_length %d exceeds max_blocks * sparse_block_size", total);
  if (total < P.S)
    return fail(KVATTN_ERR_INVALID_ARG, "total_sequence_length %d < sequence_length %d", total, P.S);
  // token generation (SparseAttention page, Description and Inputs table):
  // the new rows follow a past of key_total_sequence_lengths[b] - S rows
  P.generation = total != P.S;
  P.rotary = a->do_rotary == 1;
  if (P.rotary) {
    const kvattn_tensor& cs = in[SPARSE_IN_COS_CACHE];
    const kvattn_tensor& sn = in[SPARSE_IN_SIN_CACHE];
    if (!has(cs) || !has(sn)) return fail(KVATTN_ERR_INVALID_ARG, "do_rotary needs cos_cache and sin_cache");
    CHECK(check(cs, "cos_cache", dt, 2, {-1, -1}));
    CHECK(check(sn, "sin_cache", dt, 2, {cs.dims[0], cs.dims[1]}));
    P.rot_half = (int)cs.dims[1];
    if (P.rot_half < 8 || P.rot_half % 8 || 2 * P.rot_half > P.H)
      return fail(KVATTN_ERR_INVALID_ARG, "rotary width %d must be a multiple of 8 and at most head_size/2", P.rot_half);
    if (cs.dims[0] < total) return fail(KVATTN_ERR_INVALID_ARG, "cos_cache rows %lld < total_sequence_length %d", (long long)cs.dims[0], total);
  }
  const kvattn_tensor& o = out[SPARSE_OUT_OUTPUT];
  if (!has(o)) return fail(KVATTN_ERR_INVALID_ARG, "output is required");
  CHECK(check(o, "output", dt, 3, {P.B, P.S, (int64_t)P.N * P.H}));
  if ((has(out[SPARSE_OUT_PRESENT_KEY]) && out[SPARSE_OUT_PRESENT_KEY].data != pk.data) ||
      (has(out[SPARSE_OUT_PRESENT_VALUE]) && out[SPARSE_OUT_PRESENT_VALUE].data != pv.data))
    return fail(KVATTN_ERR_INVALID_ARG, "the present caches are the past buffers updated in place");
  P.ws_cnt = 0;
  P.ws_q = 0;  // the flash kernel rotates the queries as it loads them
  P.ws_part = 0;
  P.waves = 0;
  // one generated token: the decode kernel, one unit per query head, over the
  // blocks of its CSR row; prep writes the rotated query to the workspace
  // (a row lists at most max_nnz entries, whatever its pointers say: both
  // bound the table)
  P.decode = P.generation && P.S == 1 && P.max_blocks <= kSparseDecodeMaxBlocks &&
             P.max_nnz <= kSparseDecodeMaxBlocks;
  if (P.decode) {
    const int64_t units = (int64_t)P.B * P.N;
    P.waves = decode_waves(units, std::min<int64_t>(total, (int64_t)P.max_nnz * bs));
    if (P.waves > (int64_t)1 << 30) return fail(KVATTN_ERR_INVALID_ARG, "sparse decode: too many units");
    P.ws_cnt = kCounterBytes;
    P.ws_q = align256((size_t)P.B * P.N * P.H * elem_size(dt));
    P.ws_part = align256((size_t)(P.waves / 2) * (P.HP + 4) * sizeof(float));
  }
  P.ws_total = P.ws_cnt + P.ws_q + P.ws_part;
  return KVATTN_OK;
}

int sparse_run(const sparse_attrs* a, const kvattn_tensor* in, const kvattn_tensor* out,
               const SparsePlan& P, void* ws, hipStream_t st) {
  const DType dt = to_dtype(P.dt);
  const int64_t width = in[SPARSE_IN_QUERY].dims[2];
  PrepParams pp{};
  pp.q = in[SPARSE_IN_QUERY].data;
  pp.q_stride = width;
  if (P.packed_qkv) {
    pp.k = pp.v = in[SPARSE_IN_QUERY].data;
    pp.k_stride = pp.v_stride = width;
    pp.k_off = (int64_t)P.N * P.H;
    pp.v_off = (int64_t)(P.N + P.kvN) * P.H;
  } else {
    pp.k = in[SPARSE_IN_KEY].data;
    pp.v = in[SPARSE_IN_VALUE].data;
    pp.k_stride = pp.v_stride = (int64_t)P.kvN * P.H;
  }
  pp.q_out = nullptr;
  pp.kc = in[SPARSE_IN_PAST_KEY].data;
  pp.vc = in[SPARSE_IN_PAST_VALUE].data;
  if (P.rotary) {
    pp.cos = in[SPARSE_IN_COS_CACHE].data;
    pp.sin = in[SPARSE_IN_SIN_CACHE].data;
    pp.rot_half = P.rot_half;
    pp.rot_rows = (int)in[SPARSE_IN_COS_CACHE].dims[0];
    pp.interleaved = a->rotary_interleaved == 1;
  }
  pp.lens = static_cast<const int32_t*>(in[SPARSE_IN_KEY_TOTAL_SEQUENCE_LENGTHS].data);
  pp.pos_mode = P.generation ? 2 : 0;  // past_b = key_total[b] - S
  pp.B = P.B; pp.S = P.S; pp.N = P.N; pp.kvN = P.kvN; pp.H = P.H; pp.cap = P.cap;
  pp.write_q = P.decode ? 1 : 0;
  void* q_ws = P.decode ? static_cast<char*>(ws) + P.ws_cnt : nullptr;  // rotated query
  pp.q_out = q_ws;
  pp.write_kv = 1;
  pp.win_cap = 0;
  CHECK(hip_status(profiled(KVATTN_PROFILE_PREP, st, [&] { return launch_prep(dt, pp, st); }),
                   "prep launch"));

  if (P.decode) {
    DecodeParams d{};
    d.q = q_ws;
    d.k_new = d.v_new = nullptr;  // prep wrote the new rows
    d.kc = in[SPARSE_IN_PAST_KEY].data;
    d.vc = in[SPARSE_IN_PAST_VALUE].data;
    d.lens = static_cast<const int32_t*>(in[SPARSE_IN_KEY_TOTAL_SEQUENCE_LENGTHS].data);
    d.len_mode = 3;
    d.window = -1;
    d.out = out[SPARSE_OUT_OUTPUT].data;
    d.counters = static_cast<int*>(ws);
    d.part = reinterpret_cast<float*>(static_cast<char*>(ws) + P.ws_cnt + P.ws_q);
    d.B = P.B; d.N = P.N; d.kvN = P.N; d.H = P.H; d.cap = P.cap;
    d.kv_div = P.N / P.kvN;
    d.scale = resolve_scale(a->scale, P.H);
    d.head_groups = 1; d.hpw = 1; d.waves = (int)P.waves;
    d.split = (int64_t)d.B * d.kvN * d.head_groups <= kCounterSlots;
    d.csr_rp = static_cast<const int32_t*>(in[SPARSE_IN_BLOCK_ROW_INDICES].data);
    d.csr_cols = static_cast<const int32_t*>(in[SPARSE_IN_BLOCK_COL_INDICES].data);
    d.rp_stride = P.max_blocks + 1;
    d.cols_stride = P.max_nnz;
    d.num_layout = P.L;
    d.block = P.bs;
    d.max_blocks = P.max_blocks;
    CHECK(hip_status(profiled(KVATTN_PROFILE_DECODE, st, [&] { return launch_decode(dt, P.HP, d, st); }),
                     "decode launch"));
    return ok();
  }

  FlashParams f{};
  f.q = in[SPARSE_IN_QUERY].data;
  f.q_s = width;
  f.cos = pp.cos;
  f.sin = pp.sin;
  f.rot_half = pp.rot_half;
  f.rot_rows = pp.rot_rows;
  f.interleaved = pp.interleaved;
  f.q_b = f.q_s * P.S;
  f.q_h = P.H;
  f.kc = in[SPARSE_IN_PAST_KEY].data;
  f.vc = in[SPARSE_IN_PAST_VALUE].data;
  f.k_j = P.H;
  f.k_h = (int64_t)P.cap * P.H;
  f.k_b = f.k_h * P.kvN;
  f.out = out[SPARSE_OUT_OUTPUT].data;
  f.o_s = (int64_t)P.N * P.H;
  f.o_b = f.o_s * P.S;
  f.o_h = P.H;
  f.causal = 1;
  f.window = -1;
  f.rp = static_cast<const int32_t*>(in[SPARSE_IN_BLOCK_ROW_INDICES].data);
  f.cols = static_cast<const int32_t*>(in[SPARSE_IN_BLOCK_COL_INDICES].data);
  f.rp_stride = P.max_blocks + 1;
  f.cols_stride = P.max_nnz;
  f.num_layout = P.L;
  f.block = P.bs;
  f.max_blocks = P.max_blocks;
  f.key_total = static_cast<const int32_t*>(in[SPARSE_IN_KEY_TOTAL_SEQUENCE_LENGTHS].data);
  f.has_past = P.generation;
  f.kv_rows = P.cap;
  f.B = P.B; f.S = P.S; f.N = P.N; f.kvN = P.kvN; f.H = P.H;
  f.scale = resolve_scale(a->scale, P.H);
  f.heads_per_wg = 1;
  f.rows_per_wg = P.bs >= 128 ? 128 : P.bs;
  f.mode = kCsr;
  // token generation: row blocks aligned to absolute positions need one more
  const int gx = (P.S + f.rows_per_wg - 1) / f.rows_per_wg + (P.generation ? 1 : 0);
  CHECK(hip_status(profiled(KVATTN_PROFILE_FLASH, st,
                            [&] { return launch_flash(dt, P.HP, f, gx, P.N, P.B, st); }),
                   "flash launch"));
  return ok();
}

// ===========================================================================
// PackedAttention
// ===========================================================================
constexpr int kPackedTile = 128;

struct PackedPlan {
  int T, D, C, B, S, N, H, HP, dt, qh, kh, vh;
  size_t ws_y, ws_bounds, ws_work, ws_total;  // after the counter bytes
};

int packed_validate(const packed_attrs* a, const kvattn_tensor* in, int n_in,
                    const kvattn_tensor* out, int n_out, PackedPlan& P) {
  if (!a || !in || !out) return fail(KVATTN_ERR_INVALID_ARG, "packed_attention: null argument");
  if (n_in != PACKED_NUM_INPUTS || n_out != PACKED_NUM_OUTPUTS)
    return fail(KVATTN_ERR_INVALID_ARG, "packed_attention: expected %d inputs and %d outputs", PACKED_NUM_INPUTS, PACKED_NUM_OUTPUTS);
  const kvattn_tensor& x = in[PACKED_IN_INPUT];
  if (!has(x)) return fail(KVATTN_ERR_INVALID_ARG, "input is required");
  if (x.dtype != KVATTN_DT_F16 && x.dtype != KVATTN_DT_F32)
    return fail(KVATTN_ERR_UNSUPPORTED, "input dtype %d: only float16 and float32", x.dtype);
  const int dt = x.dtype;
  P.dt = dt;
  CHECK(check(x, "input", dt, 2, {-1, -1}));
  P.T = (int)x.dims[0];
  P.D = (int)x.dims[1];
  const kvattn_tensor& w = in[PACKED_IN_WEIGHTS];
  const kvattn_tensor& bias = in[PACKED_IN_BIAS];
  if (!has(w) || !has(bias)) return fail(KVATTN_ERR_INVALID_ARG, "weights and bias are required");
  CHECK(check(w, "weights", dt, 2, {P.D, -1}));
  P.C = (int)w.dims[1];
  CHECK(check(bias, "bias", dt, 1, {P.C}));
  P.N = a->num_heads;
  if (P.N <= 0) return fail(KVATTN_ERR_INVALID_ARG, "num_heads must be positive");
  const int* hs = a->qkv_hidden_sizes;
  if (hs[0] == 0 && hs[1] == 0 && hs[2] == 0) {
    if (P.C % 3) return fail(KVATTN_ERR_INVALID_ARG, "bias length %d does not split in three", P.C);
    P.qh = P.kh = P.vh = P.C / 3;
  } else {
    P.qh = hs[0]; P.kh = hs[1]; P.vh = hs[2];
    if (P.qh <= 0 || P.kh <= 0 || P.vh <= 0 || P.qh + P.kh + P.vh != P.C)
      return fail(KVATTN_ERR_INVALID_ARG, "qkv_hidden_sizes must be positive and sum to the weight columns");
  }
  if (P.qh != P.kh) return fail(KVATTN_ERR_INVALID_ARG, "q_hidden must equal k_hidden");
  if (P.qh % P.N || P.vh % P.N) return fail(KVATTN_ERR_INVALID_ARG, "hidden sizes must be divisible by num_heads");
  if (P.vh != P.qh) return fail(KVATTN_ERR_UNSUPPORTED, "a value head size different from the query head size is not implemented on the GPU");
  P.H = P.qh / P.N;
  CHECK(check_head_size(P.H, "packed_attention"));
  P.HP = padded_head(P.H);
  if (P.D <= 0) return fail(KVATTN_ERR_INVALID_ARG, "input hidden size must be positive");
  if (P.D % 8 || P.C % 8) return fail(KVATTN_ERR_UNSUPPORTED, "input hidden %d and weight columns %d must be multiples of 8", P.D, P.C);
  // the projection reads the weights through one buffer resource (32-bit offsets)
  if ((int64_t)P.D * P.C * (dt == KVATTN_DT_F32 ? 4 : 2) > INT32_MAX)
    return fail(KVATTN_ERR_UNSUPPORTED, "weights of %d x %d elements exceed 2 GiB", P.D, P.C);
  const kvattn_tensor& to = in[PACKED_IN_TOKEN_OFFSET];
  const kvattn_tensor& cum = in[PACKED_IN_CUMULATIVE_SEQUENCE_LENGTH];
  if (!has(to) || !has(cum)) return fail(KVATTN_ERR_INVALID_ARG, "token_offset and cumulative_sequence_length are required");
  CHECK(check(to, "token_offset", KVATTN_DT_I32, 2, {-1, -1}));
  P.B = (int)to.dims[0];
  P.S = (int)to.dims[1];
  CHECK(check(cum, "cumulative_sequence_length", KVATTN_DT_I32, 1, {(int64_t)P.B + 1}));
  if ((int64_t)P.T > (int64_t)P.B * P.S) return fail(KVATTN_ERR_INVALID_ARG, "token_count %d exceeds batch * sequence_length", P.T);
  if (P.B < 1 || P.B > 4096) return fail(KVATTN_ERR_UNSUPPORTED, "batch %d outside 1..4096", P.B);
  const kvattn_tensor& ab = in[PACKED_IN_ATTENTION_BIAS];
  if (has(ab)) {
    CHECK(check(ab, "attention_bias", dt, 4, {-1, -1, P.S, P.S}));
    if (ab.dims[0] != 1 && ab.dims[0] != P.B) return fail(KVATTN_ERR_INVALID_ARG, "attention_bias dim 0 must be 1 or batch");
    if (ab.dims[1] != 1 && ab.dims[1] != P.N) return fail(KVATTN_ERR_INVALID_ARG, "attention_bias dim 1 must be 1 or num_heads");
  }
  const kvattn_tensor& o = out[PACKED_OUT_OUTPUT];
  if (!has(o)) return fail(KVATTN_ERR_INVALID_ARG, "output is required");
  CHECK(check(o, "output", dt, 2, {P.T, P.vh}));
  P.ws_y = align256((size_t)P.T * P.C * elem_size(dt));
  P.ws_bounds = align256((size_t)2 * P.B * sizeof(int32_t));
  const size_t items = (size_t)P.B * ((P.S + kPackedTile - 1) / kPackedTile);
  P.ws_work = align256((1 + 2 * items) * sizeof(int32_t));
  P.ws_total = kCounterBytes + P.ws_y + P.ws_bounds + P.ws_work;
  return KVATTN_OK;
}

int packed_run(const packed_attrs* a, const kvattn_tensor* in, const kvattn_tensor* out,
               const PackedPlan& P, void* ws, hipStream_t st) {
  const DType dt = to_dtype(P.dt);
  char* wsb = static_cast<char*>(ws) + kCounterBytes;
  void* y = wsb;
  int32_t* bounds = reinterpret_cast<int32_t*>(wsb + P.ws_y);
  int32_t* work = reinterpret_cast<int32_t*>(wsb + P.ws_y + P.ws_bounds);

  PackedSchedParams sp{};
  sp.cum = static_cast<const int32_t*>(in[PACKED_IN_CUMULATIVE_SEQUENCE_LENGTH].data);
  sp.bounds = bounds;
  sp.work = work;
  sp.B = P.B; sp.T = P.T; sp.pad_seq = P.S; sp.tile = kPackedTile;

  GemmParams g{};
  if (P.B <= kGemmSchedMaxB) {
    g.with_sched = 1;  // the GEMM launch builds the schedule in one extra workgroup
    g.sched = sp;
  } else {
    CHECK(hip_status(launch_packed_sched(sp, st), "schedule launch"));
  }
  g.x = in[PACKED_IN_INPUT].data;
  g.w = in[PACKED_IN_WEIGHTS].data;
  g.bias = in[PACKED_IN_BIAS].data;
  g.y = y;
  g.M = P.T; g.K = P.D; g.Ncol = P.C;
  g.head_dim = P.H;  // Q, K, V head-major: every head's rows contiguous for the attention tiles
  CHECK(hip_status(profiled(KVATTN_PROFILE_GEMM, st, [&] { return launch_qkv_gemm(dt, g, st); }),
                   "qkv gemm launch"));

  FlashParams f{};
  const size_t esz = elem_size(P.dt);
  const int64_t head_el = (int64_t)P.T * P.H;  // elements of one head's rows
  f.q = y;
  f.q_s = P.H;
  f.q_h = head_el;
  f.kc = static_cast<char*>(y) + (size_t)P.N * head_el * esz;
  f.vc = static_cast<char*>(y) + (size_t)2 * P.N * head_el * esz;
  f.k_j = P.H;
  f.k_h = head_el;
  f.out = out[PACKED_OUT_OUTPUT].data;
  f.o_s = P.vh;
  f.o_h = P.H;
  const kvattn_tensor& ab = in[PACKED_IN_ATTENTION_BIAS];
  if (has(ab)) {
    f.bias = ab.data;
    f.bias_ss = P.S;
    f.bias_cols = P.S;
    f.bias_sh = ab.dims[1] > 1 ? (int64_t)P.S * P.S : 0;
    f.bias_sb = ab.dims[0] > 1 ? (int64_t)ab.dims[1] * P.S * P.S : 0;
    f.token_offset = static_cast<const int32_t*>(in[PACKED_IN_TOKEN_OFFSET].data);
    f.pad_seq = P.S;
  }
  f.lens = bounds;
  f.work = work;
  f.kv_rows = P.T;
  f.B = P.B; f.S = P.S; f.N = P.N; f.kvN = P.N; f.H = P.H;
  f.scale = resolve_scale(a->scale, P.H);
  f.heads_per_wg = 1;
  f.rows_per_wg = kPackedTile;
  f.mode = kVarlen;
  const int gx = P.B * ((P.S + kPackedTile - 1) / kPackedTile);
  CHECK(hip_status(profiled(KVATTN_PROFILE_FLASH, st,
                            [&] { return launch_flash(dt, P.HP, f, gx, P.N, 1, st); }),
                   "flash launch"));
  return ok();
}

int check_ws(size_t need, void* ws, size_t bytes) {
  if (need > 0 && (ws == nullptr || bytes < need))
    return fail(KVATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? bytes : (size_t)0);
  return KVATTN_OK;
}

// ---------------------------------------------------------------------------
// Library-held scratch for gqa_attention_noalloc: a file-scope device array,
// one copy per GPU, that serves as the workspace.  Host code never uses the
// array's name as an address: each device's copy is looked up once, with that
// device current, and kept in g_scratch_ptr.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)KVATTN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Zero words [0, n) (the arrival counters); a kernel rather than a memset so
// that a call captured into a graph records no memset node.
__global__ void clear_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The current device's scratch.  The first call on a device looks the array
// up and clears its counter bytes on `st` (they start zero and every call
// leaves them zero).
int scratch_for_device(void** out, hipStream_t st) {
  int dev = -1;
  CHECK(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KVATTN_ERR_UNSUPPORTED, "gqa_attention_noalloc: device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    CHECK(hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (ptr == nullptr) return fail(KVATTN_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
    const int words = (int)(kCounterBytes / sizeof(uint32_t));
    hipLaunchKernelGGL(clear_words_kernel, dim3((words + 255) / 256), dim3(256), 0, st,
                       static_cast<uint32_t*>(ptr), words);
    CHECK(hip_status(hipGetLastError(), "scratch counter clear launch"));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KVATTN_OK;
}

}  // namespace

// Compute units of the current device, for the launch code of the kernels.
int kvattn::cu_count() { return device_cu_count(); }

// ===========================================================================
// exported symbols
// ===========================================================================
extern "C" {

const char* kvattn_status_string(int32_t s) {
  switch (s) {
    case KVATTN_OK: return "ok";
    case KVATTN_ERR_INVALID_ARG: return "invalid argument";
    case KVATTN_ERR_UNSUPPORTED: return "unsupported";
    case KVATTN_ERR_WORKSPACE: return "workspace too small";
    case KVATTN_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* kvattn_last_error(void) { return g_last_error.c_str(); }

int32_t kvattn_version(void) { return 200; }

void kvattn_profile_events(void* start, void* stop, int32_t kind) {
  g_prof_start = static_cast<hipEvent_t>(start);
  g_prof_stop = static_cast<hipEvent_t>(stop);
  g_prof_kind = (start && stop) ? kind : 0;
}

int32_t kvattn_set_decode_split(int32_t waves_per_cu) {
  const int32_t prev = g_decode_waves_per_cu;
  if (waves_per_cu < 0 || waves_per_cu > 32)
    return fail(KVATTN_ERR_INVALID_ARG, "kvattn_set_decode_split: %d waves per compute unit (0..32)", waves_per_cu);
  g_decode_waves_per_cu = waves_per_cu;
  ok();
  return prev;
}

void gqa_attrs_default(gqa_attrs* a) {
  if (!a) return;
  std::memset(a, 0, sizeof(*a));
  a->causal = 1;
  a->local_window_size = -1;
  a->qk_norm_epsilon = 1e-6f;
  a->smooth_softmax = -1;
}

void dmmha_attrs_default(dmmha_attrs* a) {
  if (!a) return;
  std::memset(a, 0, sizeof(*a));
  a->mask_filter_value = -10000.f;
}

void sparse_attrs_default(sparse_attrs* a) {
  if (!a) return;
  std::memset(a, 0, sizeof(*a));
}

void packed_attrs_default(packed_attrs* a) {
  if (!a) return;
  std::memset(a, 0, sizeof(*a));
}

int32_t gqa_attention_workspace_size(const gqa_attrs* a, const kvattn_tensor* in, int32_t n_in,
                                     int32_t total, const kvattn_tensor* out, int32_t n_out,
                                     size_t* bytes) {
  if (!bytes) return fail(KVATTN_ERR_INVALID_ARG, "workspace_bytes is null");
  GqaPlan P{};
  CHECK(gqa_validate(a, in, n_in, total, out, n_out, P));
  *bytes = P.ws_total;
  return ok();
}

int32_t gqa_attention(const gqa_attrs* a, const kvattn_tensor* in, int32_t n_in, int32_t total,
                      const kvattn_tensor* out, int32_t n_out, void* ws, size_t ws_bytes,
                      void* stream) {
  GqaPlan P{};
  CHECK(gqa_validate(a, in, n_in, total, out, n_out, P));
  CHECK(check_ws(P.ws_total, ws, ws_bytes));
  // no new token still copies the past rows into a separate present buffer
  if (P.B == 0 || (P.S == 0 && !(P.has_past && !P.shared))) return ok();
  return gqa_run(a, in, out, P, ws, static_cast<hipStream_t>(stream));
}

int32_t gqa_attention_noalloc(const gqa_attrs* a, const kvattn_tensor* in, int32_t n_in,
                              int32_t total, const kvattn_tensor* out, int32_t n_out,
                              void* stream) {
  GqaPlan P{};
  CHECK(gqa_validate(a, in, n_in, total, out, n_out, P));
  if (P.ws_total > kScratchBytes)
    return fail(KVATTN_ERR_WORKSPACE,
                "gqa_attention_noalloc: this call needs %zu bytes of scratch, the library holds %zu "
                "(use gqa_attention with a workspace)", P.ws_total, kScratchBytes);
  if (P.B == 0 || (P.S == 0 && !(P.has_past && !P.shared))) return ok();
  const hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (P.ws_total > 0) CHECK(scratch_for_device(&ws, st));
  return gqa_run(a, in, out, P, ws, st);
}

int32_t decode_mha_workspace_size(const dmmha_attrs* a, const kvattn_tensor* in, int32_t n_in,
                                  const kvattn_tensor* out, int32_t n_out, size_t* bytes) {
  if (!bytes) return fail(KVATTN_ERR_INVALID_ARG, "workspace_bytes is null");
  DmmhaPlan P{};
  CHECK(dmmha_validate(a, in, n_in, out, n_out, P));
  *bytes = P.ws_total;
  return ok();
}

int32_t decode_mha(const dmmha_attrs* a, const kvattn_tensor* in, int32_t n_in,
                   const kvattn_tensor* out, int32_t n_out, void* ws, size_t ws_bytes,
                   void* stream) {
  DmmhaPlan P{};
  CHECK(dmmha_validate(a, in, n_in, out, n_out, P));
  CHECK(check_ws(P.ws_total, ws, ws_bytes));
  if (P.B == 0) return ok();
  return dmmha_run(a, in, out, P, ws, static_cast<hipStream_t>(stream));
}

int32_t sparse_attention_workspace_size(const sparse_attrs* a, const kvattn_tensor* in,
                                        int32_t n_in, int32_t total, const kvattn_tensor* out,
                                        int32_t n_out, size_t* bytes) {
  if (!bytes) return fail(KVATTN_ERR_INVALID_ARG, "workspace_bytes is null");
  SparsePlan P{};
  CHECK(sparse_validate(a, in, n_in, total, out, n_out, P));
  *bytes = P.ws_total;
  return ok();
}

int32_t sparse_attention(const sparse_attrs* a, const kvattn_tensor* in, int32_t n_in,
                         int32_t total, const kvattn_tensor* out, int32_t n_out, void* ws,
                         size_t ws_bytes, void* stream) {
  SparsePlan P{};
  CHECK(sparse_validate(a, in, n_in, total, out, n_out, P));
  CHECK(check_ws(P.ws_total, ws, ws_bytes));
  if (P.B == 0 || P.S == 0) return ok();
  return sparse_run(a, in, out, P, ws, static_cast<hipStream_t>(stream));
}

int32_t packed_attention_workspace_size(const packed_attrs* a, const kvattn_tensor* in,
                                        int32_t n_in, const kvattn_tensor* out, int32_t n_out,
                                        size_t* bytes) {
  if (!bytes) return fail(KVATTN_ERR_INVALID_ARG, "workspace_bytes is null");
  PackedPlan P{};
  CHECK(packed_validate(a, in, n_in, out, n_out, P));
  *bytes = P.ws_total;
  return ok();
}

int32_t packed_attention(const packed_attrs* a, const kvattn_tensor* in, int32_t n_in,
                         const kvattn_tensor* out, int32_t n_out, void* ws, size_t ws_bytes,
                         void* stream) {
  PackedPlan P{};
  CHECK(packed_validate(a, in, n_in, out, n_out, P));
  CHECK(check_ws(P.ws_total, ws, ws_bytes));
  if (P.T == 0) return ok();
  return packed_run(a, in, out, P, ws, static_cast<hipStream_t>(stream));
}

int32_t kvattn_packed_schedule(const int32_t* cum, int32_t batch, int32_t token_count,
                               int32_t padded_sequence_length, int32_t tile_rows,
                               int32_t* bounds, int32_t* work, int32_t* token_sequence,
                               int32_t* token_position, void* stream) {
  if (!cum || !bounds || !work || batch < 1 || batch > 4096 || token_count < 0 ||
      padded_sequence_length < 1 || tile_rows < 1)
    return fail(KVATTN_ERR_INVALID_ARG, "kvattn_packed_schedule: invalid argument");
  if ((token_sequence == nullptr) != (token_position == nullptr))
    return fail(KVATTN_ERR_INVALID_ARG, "token_sequence and token_position go together");
  PackedSchedParams sp{};
  sp.cum = cum;
  sp.bounds = bounds;
  sp.work = work;
  sp.tok_seq = token_sequence;
  sp.tok_pos = token_position;
  sp.B = batch; sp.T = token_count; sp.pad_seq = padded_sequence_length; sp.tile = tile_rows;
  CHECK(hip_status(launch_packed_sched(sp, static_cast<hipStream_t>(stream)), "schedule launch"));
  return ok();
}

}  // extern "C"
