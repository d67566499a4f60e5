// C-ABI entry points of libkvq: argument validation (host only, before any
// HIP call), buffer sizing, split planning and kernel dispatch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "kvq.h"
#include "kvq_internal.h"

namespace {

using kvq::CacheArgs;
using kvq::TensorArgs;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool is_pow2_group(int g) { return g == 32 || g == 64 || g == 128; }

struct Shape {
  long long B, H, S;
};

// Structural checks shared by every entry point (no pointer checks).
kvq_status check_config(const kvq_cache* c) {
  if (!c) return KVQ_ERR_INVALID_ARG;
  if (c->batch < 1 || c->kv_heads < 1 || c->max_seq < 64) return KVQ_ERR_INVALID_ARG;
  if (c->max_seq % 64) return KVQ_ERR_INVALID_ARG;
  if (c->head_dim != KVQ_HEAD_DIM) return KVQ_ERR_UNSUPPORTED;
  const kvq_tensor& k = c->k;
  const kvq_tensor& v = c->v;
  if (c->page_tokens != 0) {
    if (c->page_tokens != 64 && c->page_tokens != 128 && c->page_tokens != 256) return KVQ_ERR_INVALID_ARG;
    if (c->max_seq % c->page_tokens || c->num_pages < 1) return KVQ_ERR_INVALID_ARG;
    // every mode: uniform caches (a channel-axis K's fp16 tail stays per
    // sequence), Oaken's dense body (its sparse lists stay per sequence),
    // chunk-mixed class pools (one block-table row per class and sequence;
    // page_tokens is a multiple of chunk_tokens) and DSQ's groups (its fp16
    // tails stay per sequence)
  }
  switch (c->mode) {
    case KVQ_MODE_UNIFORM: {
      for (const kvq_tensor* t : {&k, &v}) {
        if (t->bits != 8 && t->bits != 4 && t->bits != 2) return KVQ_ERR_INVALID_ARG;
        if (t->symmetric != 0 && t->symmetric != 1) return KVQ_ERR_INVALID_ARG;
        if (t->format != KVQ_FMT_INT && t->format != KVQ_FMT_E4M3 && t->format != KVQ_FMT_E5M2)
          return KVQ_ERR_INVALID_ARG;
        if (t->format != KVQ_FMT_INT && (t->bits != 8 || t->symmetric || t->axis != KVQ_AXIS_TOKEN))
          return KVQ_ERR_UNSUPPORTED;
        if (t->symmetric && t->bits != 8) return KVQ_ERR_UNSUPPORTED;
        if (t->axis != KVQ_AXIS_TOKEN && t->axis != KVQ_AXIS_CHANNEL) return KVQ_ERR_INVALID_ARG;
      }
      if (v.axis != KVQ_AXIS_TOKEN) return KVQ_ERR_UNSUPPORTED;
      if (!is_pow2_group(v.group)) return KVQ_ERR_INVALID_ARG;
      if (k.axis == KVQ_AXIS_TOKEN && !is_pow2_group(k.group)) return KVQ_ERR_INVALID_ARG;
      if (k.axis == KVQ_AXIS_CHANNEL) {
        if (k.group != 64) return KVQ_ERR_UNSUPPORTED;
        if (k.symmetric) return KVQ_ERR_UNSUPPORTED;
      }
      TensorArgs ka{}, va{};
      ka.bits = k.bits; ka.sym = k.symmetric; ka.fmt = k.format; ka.axis = k.axis; ka.group = k.group;
      va.bits = v.bits; va.sym = v.symmetric; va.fmt = v.format; va.axis = v.axis; va.group = v.group;
      if (!kvq::decode_uniform_supported(ka, va)) return KVQ_ERR_UNSUPPORTED;
      return KVQ_OK;
    }
    case KVQ_MODE_OAKEN: {
      for (const kvq_tensor* t : {&k, &v}) {
        if (t->bits != 4 || t->symmetric || t->axis != KVQ_AXIS_TOKEN || t->format != KVQ_FMT_INT)
          return KVQ_ERR_UNSUPPORTED;
        if (!is_pow2_group(t->group)) return KVQ_ERR_INVALID_ARG;
        if (!std::isfinite(t->thr[0]) || !std::isfinite(t->thr[3]) || !(t->thr[0] < t->thr[3]))
          return KVQ_ERR_INVALID_ARG;
        // below 2^31 entries: entry byte offsets within a list fit 32 bits
        if (t->sparse_cap < 0 || t->sparse_cap > 0x7FFFFFFCll) return KVQ_ERR_INVALID_ARG;
        // lists start 8-byte aligned: decode reads them four entries per load
        if (t->sparse_cap % 4) return KVQ_ERR_ALIGNMENT;
      }
      if (k.group != v.group) return KVQ_ERR_UNSUPPORTED;
      return KVQ_OK;
    }
    case KVQ_MODE_CHUNK_MIXED: {
      if (c->chunk_tokens != 16 && c->chunk_tokens != 32 && c->chunk_tokens != 64)
        return KVQ_ERR_INVALID_ARG;
      if (!is_pow2_group(k.group) || k.group != v.group) return KVQ_ERR_INVALID_ARG;
      if (k.axis != KVQ_AXIS_TOKEN || v.axis != KVQ_AXIS_TOKEN) return KVQ_ERR_UNSUPPORTED;
      if (k.format != KVQ_FMT_INT || v.format != KVQ_FMT_INT) return KVQ_ERR_UNSUPPORTED;
      return KVQ_OK;
    }
    case KVQ_MODE_DSQ: {
      if (c->dsq_sig < 1 || c->dsq_sig > 16) return KVQ_ERR_INVALID_ARG;
      if (k.group != 32 || v.group != 32) return KVQ_ERR_UNSUPPORTED;
      if (k.axis != KVQ_AXIS_TOKEN || v.axis != KVQ_AXIS_TOKEN) return KVQ_ERR_UNSUPPORTED;
      if (k.format != KVQ_FMT_INT || v.format != KVQ_FMT_INT) return KVQ_ERR_UNSUPPORTED;
      return KVQ_OK;
    }
    default:
      return KVQ_ERR_INVALID_ARG;
  }
}

kvq_tensor_bytes tensor_bytes(const kvq_cache* c, const kvq_tensor& t, bool is_k) {
  kvq_tensor_bytes r{};
  size_t B = (size_t)c->batch, S = (size_t)c->max_seq;
  const size_t B_seq = B, S_seq = S;  // per-sequence buffers keep these when paged
  const size_t H = (size_t)c->kv_heads, D = KVQ_HEAD_DIM;
  if (c->page_tokens) {  // pools of pages: (B, S) rows become (num_pages, page_tokens)
    B = (size_t)c->num_pages;
    S = (size_t)c->page_tokens;
  }
  const size_t ng = D / (size_t)t.group;
  switch (c->mode) {
    case KVQ_MODE_UNIFORM:
      r.codes = B * H * S * D * (size_t)t.bits / 8;
      if (is_k && t.axis == KVQ_AXIS_CHANNEL) {
        r.scale = B * H * (S / 64) * D * 4;
        r.zero = B * H * (S / 64) * D;
        // fp16 residual tail: the incomplete 64-token block (per sequence, paged or not)
        r.codes16 = B_seq * H * 64 * D * 2;
      } else {
        r.scale = B * H * S * ng * 4;
        r.zero = (t.symmetric || t.format != KVQ_FMT_INT) ? 0 : B * H * S * ng;
      }
      break;
    case KVQ_MODE_OAKEN:
      r.codes = B * H * S * D / 2;
      r.scale = B * H * S * ng * 4;
      r.zero = B * H * S * ng;
      r.oscale = B * H * S * ng * 4;
      // the sparse lists are per (sequence, head) CSR, paged or not
      r.rowptr = B_seq * H * (S_seq + 1) * 4;
      r.sparse = B_seq * H * (size_t)t.sparse_cap * 2;
      break;
    case KVQ_MODE_CHUNK_MIXED:
      // 64 spare rows: decode tiles of 32 tokens over the waiting chunk of the
      // last (b, h) may reach up to 16 rows past it when chunks hold 16 tokens
      r.codes16 = (B * H * S + 64) * D * 2;
      r.codes = B * H * S * D / 2;
      r.scale = B * H * S * ng * 4;
      r.zero = B * H * S * ng;
      r.codes2 = B * H * S * D / 4;
      r.scale2 = B * H * S * ng * 4;
      r.zero2 = B * H * S * ng;
      break;
    case KVQ_MODE_DSQ: {
      // per 64-token group: 16 significant-row slots (int8, channel scales)
      // and 64 other-row slots (INT2, groups of 32 channels)
      const size_t Q = S / 64;
      r.codes = B * H * Q * 16 * D;
      r.scale = B * H * Q * D * 4;
      r.codes2 = B * H * Q * 64 * D / 4;
      r.scale2 = B * H * Q * 64 * (D / 32) * 4;
      r.zero2 = B * H * Q * 64 * (D / 32);
      // the group being appended (per sequence, paged or not): fp16 rows, and
      // (K) the tokens' scores
      r.codes16 = B_seq * H * 64 * D * 2;
      if (is_k) r.oscale = B_seq * H * 64 * 4;
      break;
    }
  }
  return r;
}

// Every buffer the mode needs must be present and 16-byte aligned.
kvq_status check_buffers(const kvq_cache* c) {
  if (!c->status || !aligned(c->status, 4)) return c->status ? KVQ_ERR_ALIGNMENT : KVQ_ERR_INVALID_ARG;
  for (int which = 0; which < 2; ++which) {
    const kvq_tensor& t = which ? c->v : c->k;
    const kvq_tensor_bytes nb = tensor_bytes(c, t, which == 0);
    const void* ptrs[10] = {t.codes, t.scale, t.zero, t.oscale, t.rowptr,
                            t.sparse, t.codes16, t.codes2, t.scale2, t.zero2};
    const size_t sizes[10] = {nb.codes, nb.scale, nb.zero, nb.oscale, nb.rowptr,
                              nb.sparse, nb.codes16, nb.codes2, nb.scale2, nb.zero2};
    for (int i = 0; i < 10; ++i) {
      if (!sizes[i]) continue;
      if (!ptrs[i]) return KVQ_ERR_INVALID_ARG;
      if (!aligned(ptrs[i], 16)) return KVQ_ERR_ALIGNMENT;
    }
  }
  if (c->mode == KVQ_MODE_CHUNK_MIXED) {
    if (!c->perm || !c->seg) return KVQ_ERR_INVALID_ARG;
    if (!aligned(c->perm, 4) || !aligned(c->seg, 16)) return KVQ_ERR_ALIGNMENT;
  }
  if (c->page_tokens) {
    if (!c->block_table) return KVQ_ERR_INVALID_ARG;
    if (!aligned(c->block_table, 4)) return KVQ_ERR_ALIGNMENT;
  }
  if (c->mode == KVQ_MODE_DSQ) {
    if (!c->dsq_mask) return KVQ_ERR_INVALID_ARG;
    if (!aligned(c->dsq_mask, 8)) return KVQ_ERR_ALIGNMENT;
  }
  return KVQ_OK;
}

TensorArgs tensor_args(const kvq_tensor& t) {
  TensorArgs a;
  a.bits = t.bits;
  a.sym = t.symmetric;
  a.fmt = t.format;
  a.axis = t.axis;
  a.group = t.group;
  a.thr_lo = t.thr[0];
  a.thr_hi = t.thr[3];
  a.sparse_cap = t.sparse_cap;
  a.codes = static_cast<uint8_t*>(t.codes);
  a.scale = t.scale;
  a.zero = t.zero;
  a.oscale = t.oscale;
  a.rowptr = t.rowptr;
  a.sparse = t.sparse;
  a.codes16 = static_cast<uint8_t*>(t.codes16);
  a.codes2 = static_cast<uint8_t*>(t.codes2);
  a.scale2 = t.scale2;
  a.zero2 = t.zero2;
  return a;
}

CacheArgs cache_args(const kvq_cache* c) {
  CacheArgs a;
  a.B = c->batch;
  a.H = c->kv_heads;
  a.S = c->max_seq;
  a.mode = c->mode;
  a.chunk_tokens = c->chunk_tokens;
  a.k = tensor_args(c->k);
  a.v = tensor_args(c->v);
  a.perm = c->perm;
  a.seg = c->seg;
  a.status = c->status;
  a.pages = c->page_tokens ? c->block_table : nullptr;
  a.ptok = c->page_tokens;
  a.npages = c->num_pages;
  a.dsq_sig = c->mode == KVQ_MODE_DSQ ? c->dsq_sig : 0;
  a.dsq_mask = reinterpret_cast<unsigned long long*>(c->mode == KVQ_MODE_DSQ ? c->dsq_mask : nullptr);
  return a;
}

kvq_status from_hip(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

// Split planning.  One workgroup (4 waves) per (b, kv head, query tile)
// already fills the GPU when there are at least kWideUnits of them; fewer
// units are split along the sequence towards one round of resident
// workgroups (256 CUs x the workgroups a CU holds at the kernel's register
// use: 4 for one query row, 3 for four, 2 for sixteen; 4 for four rows with
// channel-axis K of at most 4 bits and two V groups, whose kernel is built
// for four waves per SIMD), and the partials merged by a second kernel.
constexpr long long kWideUnits = 384;
long long target_groups(const kvq_cache* c, int qr) {
  if (qr == 4 && c->mode == KVQ_MODE_UNIFORM && c->k.axis == KVQ_AXIS_CHANNEL && c->k.bits <= 4 &&
      c->v.group == 64)
    return 1024;
  return qr == 1 ? 1024 : (qr == 4 ? 768 : 512);
}

struct Plan {
  int G, qr, qtiles, num_splits, split_len;
};

kvq_status plan_decode(const kvq_cache* c, int q_heads, int max_len, int num_splits, Plan* p) {
  if (q_heads < 1 || q_heads % c->kv_heads) return KVQ_ERR_INVALID_ARG;
  if (num_splits < 0) return KVQ_ERR_INVALID_ARG;
  p->G = q_heads / c->kv_heads;
  p->qr = p->G == 1 ? 1 : (p->G <= 4 ? 4 : kvq::kMaxQR);
  p->qtiles = (p->G + p->qr - 1) / p->qr;
  const long long units = (long long)c->batch * c->kv_heads * p->qtiles;
  long long length, min_piece, align;
  if (c->mode == KVQ_MODE_CHUNK_MIXED) {
    length = c->max_seq / c->chunk_tokens;  // chunk slots
    min_piece = 256 / c->chunk_tokens;
    align = 1;
  } else {
    if (max_len < 0) return KVQ_ERR_INVALID_ARG;
    if (max_len > c->max_seq) return KVQ_ERR_CAPACITY;
    length = max_len;
    min_piece = 256;
    align = 64;
  }
  if (length <= 0) {
    p->num_splits = 1;
    p->split_len = (int)align;
    return KVQ_OK;
  }
  long long ns = num_splits;
  if (ns == 0) {
    const long long groups = target_groups(c, p->qr);
    ns = units >= kWideUnits ? 1 : (groups + units - 1) / units;
    const long long most = (length + min_piece - 1) / min_piece;
    if (ns > most) ns = most;
  }
  if (ns < 1) ns = 1;
  if (ns > length) ns = length;
  long long piece = (length + ns - 1) / ns;
  piece = (piece + align - 1) / align * align;
  ns = (length + piece - 1) / piece;
  if (ns > 65535) return KVQ_ERR_UNSUPPORTED;
  p->num_splits = (int)ns;
  p->split_len = (int)piece;
  return KVQ_OK;
}

// Decode workspace: the split partials (when the plan splits), then for
// OAKEN the K outer-value score shares [batch][q_heads][max_len], from a
// 256-byte aligned offset.
size_t partials_bytes(const kvq_cache* c, int q_heads, const Plan& p) {
  if (p.num_splits <= 1) return 0;
  return (size_t)c->batch * (size_t)q_heads * (size_t)p.num_splits * kvq::kPartStride * sizeof(float);
}
size_t oak_ksc_offset(const kvq_cache* c, int q_heads, const Plan& p) {
  return (partials_bytes(c, q_heads, p) + 255) & ~(size_t)255;
}
size_t workspace_for(const kvq_cache* c, int q_heads, int max_len, const Plan& p) {
  if (c->mode != KVQ_MODE_OAKEN || max_len <= 0) return partials_bytes(c, q_heads, p);
  return oak_ksc_offset(c, q_heads, p) + (size_t)c->batch * (size_t)q_heads * (size_t)max_len * sizeof(float);
}

// Workspace of kvq_decode_attn_noalloc: a fixed array in the device
// image (each device holds its own copy).  Host code never passes the
// array's name to a kernel: it is a host-side stand-in, and the device
// address comes from hipGetSymbolAddress, looked up once per device with
// that device current.
__device__ __align__(256) float scratch[KVQ_STATIC_SCRATCH_BYTES / sizeof(float)];
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices] = {};

kvq_status static_scratch(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KVQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return KVQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_ERR_HIP;
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_dev[dev];
  return KVQ_OK;
}

// kvq_decode_attn with the caller's workspace, or (use_static) with the
// library's fixed per-device array; every argument check precedes the first
// HIP call.
kvq_status decode_attn(const kvq_cache* c, const void* q, int32_t q_heads, const int32_t* seq_len,
                       int32_t max_len, float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                       int32_t num_splits, void* stream, bool use_static) {
  kvq_status s = check_config(c);
  if (s != KVQ_OK) return s;
  if (!q || !out) return KVQ_ERR_INVALID_ARG;
  if (c->mode != KVQ_MODE_CHUNK_MIXED && !seq_len) return KVQ_ERR_INVALID_ARG;
  if (!std::isfinite(sm_scale)) return KVQ_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(out, 16) || (seq_len && !aligned(seq_len, 4)))
    return KVQ_ERR_ALIGNMENT;
  Plan p;
  s = plan_decode(c, q_heads, max_len, num_splits, &p);
  if (s != KVQ_OK) return s;
  const size_t need = workspace_for(c, q_heads, max_len, p);
  if (use_static) {
    if (need > KVQ_STATIC_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE;
  } else if (need) {
    if (!workspace || workspace_bytes < need) return KVQ_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return KVQ_ERR_ALIGNMENT;
  }
  s = check_buffers(c);
  if (s != KVQ_OK) return s;
  if (use_static && need) {
    float* ws = nullptr;
    s = static_scratch(&ws);
    if (s != KVQ_OK) return s;
    workspace = ws;
  }
  const CacheArgs a = cache_args(c);
  kvq::DecodeLaunch d;
  d.q = static_cast<const uint16_t*>(q);
  d.Hq = q_heads;
  d.G = p.G;
  d.qr = p.qr;
  d.qtiles = p.qtiles;
  d.seq_len = seq_len;
  d.max_len = c->mode == KVQ_MODE_CHUNK_MIXED ? c->max_seq : max_len;
  d.num_splits = p.num_splits;
  d.split_len = p.split_len;
  d.qscale = sm_scale * 1.4426950408889634f;
  d.out = out;
  d.ws = p.num_splits > 1 ? static_cast<float*>(workspace) : nullptr;
  d.oak_ksc = c->mode == KVQ_MODE_OAKEN && max_len > 0
                  ? reinterpret_cast<float*>(static_cast<char*>(workspace) + oak_ksc_offset(c, q_heads, p))
                  : nullptr;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (c->mode) {
    case KVQ_MODE_UNIFORM: e = kvq::launch_decode_uniform(a, d, st); break;
    case KVQ_MODE_OAKEN: e = kvq::launch_decode_oaken(a, d, st); break;
    case KVQ_MODE_DSQ: e = kvq::launch_decode_dsq(a, d, st); break;
    default: e = kvq::launch_decode_mixed(a, d, st); break;
  }
  if (e == hipErrorInvalidValue) return KVQ_ERR_UNSUPPORTED;
  if (e != hipSuccess) return KVQ_ERR_HIP;
  if (p.num_splits > 1) e = kvq::launch_merge(d, c->batch, st);
  return from_hip(e);
}

}  // namespace

namespace kvq {

// The (K, V) pairs go_codec in kvq_decode_uniform.hip dispatches to a kernel.
bool decode_uniform_supported(const TensorArgs& k, const TensorArgs& v) {
  if (v.axis != 0) return false;
  if (v.group != 32 && v.group != 64 && v.group != 128) return false;
  if (k.bits != v.bits || k.sym != v.sym || k.fmt != v.fmt) return false;
  if (v.fmt == 1 || v.fmt == 2) return v.bits == 8 && !v.sym && k.axis == 0 && k.group == v.group;
  if (v.sym && v.bits != 8) return false;
  if (v.bits != 8 && v.bits != 4 && v.bits != 2) return false;
  if (k.axis == 0) return k.group == v.group;
  if (k.axis == 1) return k.group == 64 && !k.sym && (k.bits == 8 || k.bits == 4);
  return false;
}

}  // namespace kvq

extern "C" {

kvq_status kvq_cache_bytes(const kvq_cache* c, kvq_cache_bytes_t* out) {
  if (!out) return KVQ_ERR_INVALID_ARG;
  const kvq_status s = check_config(c);
  if (s != KVQ_OK) return s;
  *out = kvq_cache_bytes_t{};
  out->k = tensor_bytes(c, c->k, true);
  out->v = tensor_bytes(c, c->v, false);
  if (c->mode == KVQ_MODE_CHUNK_MIXED) {
    const size_t C = (size_t)(c->max_seq / c->chunk_tokens);
    out->perm = (size_t)c->batch * C * 4;
    out->seg = (size_t)c->batch * 4 * 4;
  }
  if (c->mode == KVQ_MODE_DSQ)  // one mask per group: [B][H][S / 64], or pooled with the pages
    out->dsq_mask = c->page_tokens
                        ? (size_t)c->num_pages * (size_t)c->kv_heads * (size_t)(c->page_tokens / 64) * 8
                        : (size_t)c->batch * (size_t)c->kv_heads * (size_t)(c->max_seq / 64) * 8;
  out->status = 4;
  return KVQ_OK;
}

kvq_status kvq_quant_append(const kvq_cache* c, const void* k_new, const void* v_new, int32_t t_new,
                            const int32_t* pos, void* stream) {
  kvq_status s = check_config(c);
  if (s != KVQ_OK) return s;
  if (t_new < 0) return KVQ_ERR_INVALID_ARG;
  if (t_new > c->max_seq) return KVQ_ERR_CAPACITY;
  if (t_new == 0) return KVQ_OK;
  if ((long long)c->batch * c->kv_heads * t_new >= (1ll << 31)) return KVQ_ERR_UNSUPPORTED;  // 32-bit row index
  if (!k_new || !v_new || !pos) return KVQ_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(pos, 4)) return KVQ_ERR_ALIGNMENT;
  s = check_buffers(c);
  if (s != KVQ_OK) return s;
  const CacheArgs a = cache_args(c);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* kx = static_cast<const uint16_t*>(k_new);
  const uint16_t* vx = static_cast<const uint16_t*>(v_new);
  hipError_t e = hipSuccess;
  switch (c->mode) {
    case KVQ_MODE_UNIFORM:
      if (c->k.axis == KVQ_AXIS_CHANNEL) {
        e = kvq::launch_quant_channel(a, a.k, kx, t_new, pos, st);
        if (e == hipSuccess) e = kvq::launch_quant_token(a, a.v, true, vx, t_new, pos, st);
      } else if (a.k.bits == a.v.bits && a.k.sym == a.v.sym && a.k.fmt == a.v.fmt &&
                 a.k.group == a.v.group) {
        e = kvq::launch_quant_token_kv(a, kx, vx, t_new, pos, st);
      } else {
        e = kvq::launch_quant_token(a, a.k, false, kx, t_new, pos, st);
        if (e == hipSuccess) e = kvq::launch_quant_token(a, a.v, true, vx, t_new, pos, st);
      }
      break;
    case KVQ_MODE_OAKEN:
      if (t_new == 1 && a.k.group == a.v.group) {
        e = kvq::launch_quant_oaken_one(a, kx, vx, pos, st);
      } else {
        e = kvq::launch_quant_oaken(a, a.k, false, kx, t_new, pos, st);
        if (e == hipSuccess) e = kvq::launch_quant_oaken(a, a.v, true, vx, t_new, pos, st);
      }
      break;
    case KVQ_MODE_CHUNK_MIXED:
      if (t_new != c->max_seq) return KVQ_ERR_INVALID_ARG;
      e = kvq::launch_quant_mixed(a, a.k, false, kx, pos, st);
      if (e == hipSuccess) e = kvq::launch_quant_mixed(a, a.v, true, vx, pos, st);
      break;
    default:  // DSQ needs token scores: kvq_dsq_append
      return KVQ_ERR_INVALID_ARG;
  }
  return from_hip(e);
}

kvq_status kvq_dsq_append(const kvq_cache* c, const void* k_new, const void* v_new, const float* score,
                          int32_t t_new, const int32_t* pos, void* stream) {
  kvq_status s = check_config(c);
  if (s != KVQ_OK) return s;
  if (c->mode != KVQ_MODE_DSQ) return KVQ_ERR_INVALID_ARG;
  if (t_new < 0) return KVQ_ERR_INVALID_ARG;
  if (t_new > c->max_seq) return KVQ_ERR_CAPACITY;
  if (t_new == 0) return KVQ_OK;
  if ((long long)c->batch * c->kv_heads > 65535) return KVQ_ERR_UNSUPPORTED;
  if (!k_new || !v_new || !score || !pos) return KVQ_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(score, 4) || !aligned(pos, 4))
    return KVQ_ERR_ALIGNMENT;
  s = check_buffers(c);
  if (s != KVQ_OK) return s;
  const CacheArgs a = cache_args(c);
  return from_hip(kvq::launch_quant_dsq(a, static_cast<const uint16_t*>(k_new),
                                        static_cast<const uint16_t*>(v_new), score, t_new, pos,
                                        static_cast<hipStream_t>(stream)));
}

kvq_status kvq_reorder_chunks(const kvq_cache* c, const uint8_t* chunk_bits, int32_t n_chunks,
                              void* stream) {
  kvq_status s = check_config(c);
  if (s != KVQ_OK) return s;
  if (c->mode != KVQ_MODE_CHUNK_MIXED) return KVQ_ERR_INVALID_ARG;
  if (n_chunks != c->max_seq / c->chunk_tokens) return KVQ_ERR_INVALID_ARG;
  if (!chunk_bits || !c->perm || !c->seg || !c->status) return KVQ_ERR_INVALID_ARG;
  if (!aligned(c->perm, 4) || !aligned(c->seg, 16) || !aligned(c->status, 4)) return KVQ_ERR_ALIGNMENT;
  const CacheArgs a = cache_args(c);
  return from_hip(kvq::launch_reorder(a, chunk_bits, n_chunks, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_append_chunks(const kvq_cache* c, const void* k_new, const void* v_new, int32_t t_new,
                             const int32_t* pos, const uint8_t* new_bits, int32_t n_new, void* stream) {
  kvq_status s = check_config(c);
  if (s != KVQ_OK) return s;
  if (c->mode != KVQ_MODE_CHUNK_MIXED) return KVQ_ERR_INVALID_ARG;
  if (t_new < 0) return KVQ_ERR_INVALID_ARG;
  if (t_new > c->max_seq) return KVQ_ERR_CAPACITY;
  if (t_new == 0) return KVQ_OK;
  if (n_new < (t_new + c->chunk_tokens - 1) / c->chunk_tokens) return KVQ_ERR_INVALID_ARG;
  if (!k_new || !v_new || !pos || !new_bits) return KVQ_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(pos, 4)) return KVQ_ERR_ALIGNMENT;
  s = check_buffers(c);
  if (s != KVQ_OK) return s;
  const CacheArgs a = cache_args(c);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = kvq::launch_append_chunks(a, static_cast<const uint16_t*>(k_new),
                                           static_cast<const uint16_t*>(v_new), t_new, pos, new_bits,
                                           n_new, st);
  return from_hip(e);
}

kvq_status kvq_decode_workspace_bytes(const kvq_cache* c, int32_t q_heads, int32_t max_len,
                                      int32_t num_splits, size_t* bytes) {
  if (!bytes) return KVQ_ERR_INVALID_ARG;
  kvq_status s = check_config(c);
  if (s != KVQ_OK) return s;
  Plan p;
  s = plan_decode(c, q_heads, max_len, num_splits, &p);
  if (s != KVQ_OK) return s;
  *bytes = workspace_for(c, q_heads, max_len, p);
  return KVQ_OK;
}

kvq_status kvq_decode_attn(const kvq_cache* c, const void* q, int32_t q_heads, const int32_t* seq_len,
                           int32_t max_len, float sm_scale, float* out, void* workspace,
                           size_t workspace_bytes, int32_t num_splits, void* stream) {
  return decode_attn(c, q, q_heads, seq_len, max_len, sm_scale, out, workspace, workspace_bytes, num_splits,
                     stream, false);
}

kvq_status kvq_decode_attn_noalloc(const kvq_cache* c, const void* q, int32_t q_heads,
                                   const int32_t* seq_len, int32_t max_len, float sm_scale, float* out,
                                   int32_t num_splits, void* stream) {
  return decode_attn(c, q, q_heads, seq_len, max_len, sm_scale, out, nullptr, 0, num_splits, stream, true);
}


kvq_status kvq_chunk_bits(const double* q_emb, const double* chunk_emb, int32_t batch,
                          int32_t n_chunks, int32_t dim, double alpha, double beta, double* sims,
                          uint8_t* bits, void* stream) {
  if (batch < 0 || n_chunks < 0 || dim < 1) return KVQ_ERR_INVALID_ARG;
  if (!(alpha >= 0.0 && alpha <= 1.0 && beta >= 0.0 && beta <= 1.0)) return KVQ_ERR_INVALID_ARG;
  if (batch == 0 || n_chunks == 0) return KVQ_OK;
  if (batch > 65535) return KVQ_ERR_UNSUPPORTED;
  if (!q_emb || !chunk_emb || !bits) return KVQ_ERR_INVALID_ARG;
  if (!aligned(q_emb, 8) || !aligned(chunk_emb, 8) || (sims && !aligned(sims, 8)))
    return KVQ_ERR_ALIGNMENT;
  return from_hip(kvq::launch_chunk_bits(q_emb, chunk_emb, batch, n_chunks, dim, alpha, beta, sims,
                                         bits, static_cast<hipStream_t>(stream)));
}

kvq_status kvq_hist_f16(const void* x, int64_t n, uint64_t* hist, void* stream) {
  if (n < 0 || n > (int64_t(1) << 40)) return KVQ_ERR_INVALID_ARG;
  if (n == 0) return KVQ_OK;
  if (!x || !hist) return KVQ_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(hist, 8)) return KVQ_ERR_ALIGNMENT;
  return from_hip(kvq::launch_hist_f16(static_cast<const uint16_t*>(x), (long long)n,
                                       reinterpret_cast<unsigned long long*>(hist),
                                       static_cast<hipStream_t>(stream)));
}

kvq_status kvq_hist_percentiles(const uint64_t* hist, int32_t count, const int32_t* p_bp, float* out,
                                void* stream) {
  if (count < 0 || count > kvq::kMaxPercentiles) return KVQ_ERR_INVALID_ARG;
  if (count == 0) return KVQ_OK;
  if (!hist || !p_bp || !out) return KVQ_ERR_INVALID_ARG;
  if (!aligned(hist, 8) || !aligned(out, 4)) return KVQ_ERR_ALIGNMENT;
  kvq::PercentileList pl{};
  pl.count = count;
  for (int i = 0; i < count; ++i) {
    if (p_bp[i] < 0 || p_bp[i] > 10000) return KVQ_ERR_INVALID_ARG;
    pl.p_bp[i] = p_bp[i];
  }
  return from_hip(kvq::launch_percentiles(reinterpret_cast<const unsigned long long*>(hist), pl, out,
                                          static_cast<hipStream_t>(stream)));
}

const char* kvq_status_string(int32_t status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_CAPACITY: return "exceeds cache capacity";
    case KVQ_ERR_ALIGNMENT: return "misaligned pointer";
    case KVQ_ERR_WORKSPACE: return "decode workspace missing or too small";
    case KVQ_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
