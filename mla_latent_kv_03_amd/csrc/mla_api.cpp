// Host side of the C ABI declared in include/mla_decode.h: argument validation,
// split-count choice, workspace layout and kernel launches on the caller's stream.
// No allocation, no synchronization, no device access during validation.

#include "mla_decode.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>
#include <mutex>

#include "mla_kernels.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return -1;
  if (dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

enum class Path { kNone, kF32, kBf16, kFp8 };

Path path_of(const mla_decode_params_t& p) {
  if (p.q_dtype == MLA_DTYPE_F32 && p.kv_dtype == MLA_DTYPE_F32 && p.w_dtype == MLA_DTYPE_F32 &&
      p.out_dtype == MLA_DTYPE_F32)
    return Path::kF32;
  if (p.q_dtype == MLA_DTYPE_BF16 && p.w_dtype == MLA_DTYPE_BF16 && p.out_dtype == MLA_DTYPE_BF16) {
    if (p.kv_dtype == MLA_DTYPE_BF16) return Path::kBf16;
    if (p.kv_dtype == MLA_DTYPE_FP8_E4M3) return Path::kFp8;
  }
  return Path::kNone;
}

// Rows of (query position, head) handled by one workgroup on the MFMA paths.
int rows_per_group(const mla_decode_params_t& p) {
  if (path_of(p) == Path::kBf16) return mla::attn_heads_per_group(p.n_h);
  const int rows = p.s_q * p.n_h;
  return rows <= 128 ? rows : 128;
}

mla_status_t check_common(const mla_decode_params_t* p) {
  if (!p) return MLA_ERR_NULL;
  if (p->batch < 1 || p->s_q < 1 || p->s_q > 16 || p->n_h < 1 || p->d_c < 1 || p->d_r < 0 || p->d_v < 1)
    return MLA_ERR_SHAPE;
  if (p->page_size < 64 || p->page_size % 64 != 0 || p->num_pages < 1 || p->max_pages_per_seq < 1)
    return MLA_ERR_SHAPE;
  if ((long long)p->max_pages_per_seq * p->page_size > INT_MAX) return MLA_ERR_SHAPE;
  if (p->num_splits < 0) return MLA_ERR_SHAPE;
  if (p->c_kv_stride < p->d_c || p->k_pe_stride < p->d_r) return MLA_ERR_SHAPE;
  if (!(p->softmax_scale > 0.f) || p->softmax_scale == INFINITY) return MLA_ERR_SHAPE;
  switch (path_of(*p)) {
    case Path::kNone:
      return MLA_ERR_DTYPE;
    case Path::kF32:
      if (p->d_c > 1024 || p->d_r > 256 || p->d_v > 1024 || p->n_h > 1024) return MLA_ERR_SHAPE;
      if ((long long)p->s_q * p->n_h > 65535) return MLA_ERR_SHAPE;
      break;
    case Path::kBf16:
    case Path::kFp8: {
      if (p->d_c != 512 || p->d_r != 64 || p->d_v != 128) return MLA_ERR_SHAPE;
      if (p->n_h % 16 != 0) return MLA_ERR_SHAPE;
      if (path_of(*p) == Path::kBf16) {
        if (!(p->n_h == 16 || p->n_h == 32 || p->n_h % 64 == 0)) return MLA_ERR_SHAPE;
      } else {
        const int rows = p->s_q * p->n_h;
        if (rows > 128 && rows % 128 != 0) return MLA_ERR_SHAPE;
      }
      const int align = path_of(*p) == Path::kFp8 ? 16 : 8;  // 16-byte rows for the tile copies
      if (p->c_kv_stride % align != 0 || p->k_pe_stride % align != 0) return MLA_ERR_SHAPE;
      break;
    }
  }
  return MLA_OK;
}

int resolve_splits(const mla_decode_params_t& p) {
  if (p.num_splits > 0) return p.num_splits;
  const int cus = device_cu_count();
  if (cus <= 0) return -1;
  if (path_of(p) == Path::kF32) {
    const int rows = p.s_q * p.n_h;
    int g = (2 * cus) / rows;
    return g < 1 ? 1 : (g > 64 ? 64 : g);
  }
  const int groups = (p.s_q * p.n_h) / rows_per_group(p);
  int g = cus / groups;
  if (g >= 16) g -= g % 8;   // all row groups of a share then sit on one XCD (shared L2)
  return g < 1 ? 1 : g;
}

struct Layout {
  size_t table, lse, u, total;
  int num_slots;
};

Layout layout_of(const mla_decode_params_t& p, int G) {
  Layout l;
  l.num_slots = G + p.batch;
  const size_t rows = (size_t)l.num_slots * p.s_q * p.n_h;
  l.table = 0;
  l.lse = align256((size_t)p.batch * 2 * sizeof(int32_t));
  l.u = l.lse + align256(rows * sizeof(float));
  // partial_u: float32 on the fp32 path, bf16 on the bf16 / E4M3-cache paths.
  const size_t u_elem = path_of(p) == Path::kF32 ? sizeof(float) : 2;
  l.total = l.u + align256(rows * (size_t)p.d_c * u_elem);
  return l;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

mla_status_t launch_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

mla_status_t combine_impl(const mla_decode_params_t& p, int G, const void* workspace, const void* w_uv, void* out,
                          float* lse, hipStream_t stream) {
  const Layout l = layout_of(p, G);
  mla::CombineParams c;
  c.split_table = (const int32_t*)((const char*)workspace + l.table);
  c.part_lse = (const float*)((const char*)workspace + l.lse);
  c.part_u = (const char*)workspace + l.u;
  c.w_uv = w_uv;
  c.out = out;
  c.lse = lse;
  c.batch = p.batch;
  c.s_q = p.s_q;
  c.n_h = p.n_h;
  c.d_c = p.d_c;
  c.d_v = p.d_v;
  c.num_slots = l.num_slots;
  if (path_of(p) == Path::kF32) return launch_status(mla::launch_combine_f32(c, stream));
  return launch_status(mla::launch_combine_bf16(c, stream));
}

mla_status_t prepare_fwd(const mla_decode_params_t* params, const void* q_nope, const void* q_pe, const void* c_kv,
                         const void* k_pe, const float* kv_scale, const int32_t* block_table,
                         const int32_t* seq_lens, const void* w_uv, void* workspace, size_t workspace_bytes,
                         mla::AttnParams& a, int& G) {
  mla_status_t st = check_common(params);
  if (st != MLA_OK) return st;
  const mla_decode_params_t& p = *params;
  const Path path = path_of(p);
  if (!q_nope || !q_pe || !c_kv || !block_table || !seq_lens || !w_uv) return MLA_ERR_NULL;
  if (p.d_r > 0 && !k_pe) return MLA_ERR_NULL;
  if ((path == Path::kFp8) != (kv_scale != nullptr)) return path == Path::kFp8 ? MLA_ERR_NULL : MLA_ERR_DTYPE;
  if (path != Path::kF32) {
    if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(c_kv) || !aligned16(k_pe) || !aligned16(w_uv))
      return MLA_ERR_SHAPE;
  }
  G = resolve_splits(p);
  if (G <= 0) return MLA_ERR_UNSUPPORTED;
  const Layout l = layout_of(p, G);
  if (!workspace || workspace_bytes < l.total) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_WORKSPACE;

  a.q_nope = q_nope;
  a.q_pe = q_pe;
  a.c_kv = c_kv;
  a.k_pe = k_pe ? k_pe : c_kv;
  a.kv_scale = kv_scale;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.c_stride = p.c_kv_stride;
  a.k_stride = p.k_pe_stride;
  a.batch = p.batch;
  a.s_q = p.s_q;
  a.n_h = p.n_h;
  a.d_c = p.d_c;
  a.d_r = p.d_r;
  a.page_size = p.page_size;
  a.num_pages = p.num_pages;
  a.max_pages = p.max_pages_per_seq;
  a.max_tokens = p.max_pages_per_seq * p.page_size;
  a.num_splits = G;
  a.rows_per_group = rows_per_group(p);
  {
    const size_t elem = path == Path::kF32 ? 4 : (path == Path::kFp8 ? 1 : 2);
    a.packed_rows = (k_pe == (const char*)c_kv + (size_t)p.d_c * elem && p.c_kv_stride == p.k_pe_stride) ? 1 : 0;
  }
  a.scale_log2 = p.softmax_scale * 1.4426950408889634f;
  a.split_table = (int32_t*)((char*)workspace + l.table);
  a.part_lse = (float*)((char*)workspace + l.lse);
  a.part_u = (char*)workspace + l.u;
  a.new_c = nullptr;
  a.new_k = nullptr;
  a.new_pos = nullptr;
  a.s_new = 0;
  return MLA_OK;
}

mla_status_t launch_fwd(const mla_decode_params_t& p, const mla::AttnParams& a, int G, const void* w_uv, void* out,
                        float* lse, void* workspace, hipStream_t s) {
  const Path path = path_of(p);
  hipError_t e = path == Path::kF32 ? mla::launch_attn_f32(a, s) : mla::launch_attn_mfma(a, path == Path::kFp8, s);
  if (e != hipSuccess) return MLA_ERR_HIP;
  if (!out) return MLA_OK;
  return combine_impl(p, G, workspace, w_uv, out, lse, s);
}

mla_status_t prepare_append(const mla_decode_params_t* params, const void* c_new, const void* k_pe_new,
                            int32_t s_new, mla_dtype_t in_dtype, const int32_t* positions,
                            const int32_t* block_table, void* c_kv, void* k_pe, float* kv_scale,
                            mla::AppendParams& a) {
  if (!params) return MLA_ERR_NULL;
  const mla_decode_params_t& p = *params;
  if (p.batch < 1 || s_new < 1 || p.d_c < 1 || p.d_r < 0) return MLA_ERR_SHAPE;
  if ((long long)p.batch * s_new > INT_MAX) return MLA_ERR_SHAPE;
  if (p.page_size < 64 || p.page_size % 64 != 0 || p.num_pages < 1 || p.max_pages_per_seq < 1) return MLA_ERR_SHAPE;
  if (p.c_kv_stride < p.d_c || p.k_pe_stride < p.d_r) return MLA_ERR_SHAPE;
  if (!c_new || !positions || !block_table || !c_kv) return MLA_ERR_NULL;
  if (p.d_r > 0 && (!k_pe_new || !k_pe)) return MLA_ERR_NULL;
  int mode;
  if (p.kv_dtype == MLA_DTYPE_BF16 && in_dtype == MLA_DTYPE_BF16) mode = 0;
  else if (p.kv_dtype == MLA_DTYPE_F32 && in_dtype == MLA_DTYPE_F32) mode = 1;
  else if (p.kv_dtype == MLA_DTYPE_FP8_E4M3 && (in_dtype == MLA_DTYPE_F32 || in_dtype == MLA_DTYPE_BF16)) mode = 2;
  else return MLA_ERR_DTYPE;
  if ((mode == 2) != (kv_scale != nullptr)) return mode == 2 ? MLA_ERR_NULL : MLA_ERR_DTYPE;
  a.c_new = c_new;
  a.k_new = k_pe_new ? k_pe_new : c_new;
  a.positions = positions;
  a.block_table = block_table;
  a.c_kv = c_kv;
  a.k_pe = k_pe ? k_pe : c_kv;
  a.kv_scale = kv_scale;
  a.c_stride = p.c_kv_stride;
  a.k_stride = p.k_pe_stride;
  a.batch = p.batch;
  a.s_new = s_new;
  a.d_c = p.d_c;
  a.d_r = p.d_r;
  a.page_size = p.page_size;
  a.num_pages = p.num_pages;
  a.max_pages = p.max_pages_per_seq;
  a.in_f32 = in_dtype == MLA_DTYPE_F32;
  a.mode = mode;
  return MLA_OK;
}

// Workspace of mla_decode_fwd_noalloc: one array per device, in the code object's
// zero-initialized device memory, held until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the symbol): its
// device address is looked up once per device, with that device current, and kept.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array, or nullptr if the runtime cannot give it.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();   // leave no sticky error for the caller's next HIP call
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

namespace mla {
AttentionEvents& attention_events() {
  static thread_local AttentionEvents ev;
  return ev;
}
}  // namespace mla

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

mla_status_t mla_set_attention_events(void* start, void* stop) {
  mla::AttentionEvents& ev = mla::attention_events();
  ev.start = static_cast<hipEvent_t>(start);
  ev.stop = static_cast<hipEvent_t>(stop);
  return MLA_OK;
}

const char* mla_status_string(mla_status_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: unsupported size, stride or shape combination";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: unsupported dtype combination";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: the HIP runtime reported an error";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: no kernel for this device";
    case MLA_ERR_TOO_LARGE:
      return "MLA_ERR_TOO_LARGE: the call needs more workspace than the library's static buffer "
             "(mla_decode_noalloc_capacity() bytes) holds";
  }
  return "unknown mla_status_t";
}

int32_t mla_decode_num_splits(const mla_decode_params_t* params) {
  if (check_common(params) != MLA_OK) return -1;
  return resolve_splits(*params);
}

size_t mla_decode_workspace_size(const mla_decode_params_t* params) {
  if (check_common(params) != MLA_OK) return 0;
  const int G = resolve_splits(*params);
  if (G <= 0) return 0;
  return layout_of(*params, G).total;
}

mla_status_t mla_decode_fwd(const mla_decode_params_t* params, const void* q_nope, const void* q_pe,
                            const void* c_kv, const void* k_pe, const float* kv_scale,
                            const int32_t* block_table, const int32_t* seq_lens, const void* w_uv, void* out,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  mla::AttnParams a;
  int G = 0;
  const mla_status_t st = prepare_fwd(params, q_nope, q_pe, c_kv, k_pe, kv_scale, block_table, seq_lens, w_uv,
                                      workspace, workspace_bytes, a, G);
  if (st != MLA_OK) return st;
  return launch_fwd(*params, a, G, w_uv, out, lse, workspace, (hipStream_t)stream);
}

size_t mla_decode_noalloc_capacity(void) { return kScratchBytes; }

mla_status_t mla_decode_fwd_noalloc(const mla_decode_params_t* params, const void* q_nope, const void* q_pe,
                                    const void* c_kv, const void* k_pe, const float* kv_scale,
                                    const int32_t* block_table, const int32_t* seq_lens, const void* w_uv,
                                    void* out, float* lse, void* stream) {
  const mla_status_t st = check_common(params);
  if (st != MLA_OK) return st;
  if (!out) return MLA_ERR_NULL;
  const int G = resolve_splits(*params);
  if (G <= 0) return MLA_ERR_UNSUPPORTED;
  if (layout_of(*params, G).total > kScratchBytes) return MLA_ERR_TOO_LARGE;
  void* ws = scratch_address();
  if (!ws) return MLA_ERR_HIP;
  // Nothing in the scratch array has to start at zero: the partial-attention launch writes
  // the split table and every partial that the combine then reads.
  return mla_decode_fwd(params, q_nope, q_pe, c_kv, k_pe, kv_scale, block_table, seq_lens, w_uv, out, lse, ws,
                        kScratchBytes, stream);
}

mla_status_t mla_decode_fwd_append(const mla_decode_params_t* params, const void* c_new, const void* k_pe_new,
                                   int32_t s_new, mla_dtype_t in_dtype, const int32_t* positions,
                                   const void* q_nope, const void* q_pe, void* c_kv, void* k_pe, float* kv_scale,
                                   const int32_t* block_table, const int32_t* seq_lens, const void* w_uv,
                                   void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  // Everything is validated before anything is launched.
  mla::AppendParams ap;
  mla_status_t st = prepare_append(params, c_new, k_pe_new, s_new, in_dtype, positions, block_table, c_kv, k_pe,
                                   kv_scale, ap);
  if (st != MLA_OK) return st;
  mla::AttnParams a;
  int G = 0;
  st = prepare_fwd(params, q_nope, q_pe, c_kv, k_pe, kv_scale, block_table, seq_lens, w_uv, workspace,
                   workspace_bytes, a, G);
  if (st != MLA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const mla_decode_params_t& p = *params;
  const bool fused = path_of(p) == Path::kBf16 && p.n_h % 128 == 0 && ap.mode == 0 && s_new <= mla::kMaxFusedNew &&
                     p.d_r > 0 && aligned16(c_new) && aligned16(k_pe_new) && p.c_kv_stride % 8 == 0 &&
                     p.k_pe_stride % 8 == 0;
  if (fused) {
    a.new_c = c_new;
    a.new_k = k_pe_new;
    a.new_pos = positions;
    a.s_new = s_new;
  } else {
    st = launch_status(mla::launch_append(ap, s));
    if (st != MLA_OK) return st;
  }
  return launch_fwd(p, a, G, w_uv, out, lse, workspace, s);
}

mla_status_t mla_decode_splitkv_combine(const mla_decode_params_t* params, const void* workspace,
                                        size_t workspace_bytes, const void* w_uv, void* out, float* lse,
                                        void* stream) {
  mla_status_t st = check_common(params);
  if (st != MLA_OK) return st;
  if (!out) return MLA_ERR_NULL;
  const Path path = path_of(*params);
  if (path != Path::kF32 && ((w_uv && !aligned16(w_uv)) || !aligned16(workspace) || (!w_uv && !aligned16(out))))
    return MLA_ERR_SHAPE;
  const int G = resolve_splits(*params);
  if (G <= 0) return MLA_ERR_UNSUPPORTED;
  const Layout l = layout_of(*params, G);
  if (!workspace || workspace_bytes < l.total) return MLA_ERR_WORKSPACE;
  return combine_impl(*params, G, workspace, w_uv, out, lse, (hipStream_t)stream);
}

mla_status_t mla_paged_cache_append(const mla_decode_params_t* params, const void* c_new, const void* k_pe_new,
                                    int32_t s_new, mla_dtype_t in_dtype, const int32_t* positions,
                                    const int32_t* block_table, void* c_kv, void* k_pe, float* kv_scale,
                                    void* stream) {
  mla::AppendParams a;
  const mla_status_t st = prepare_append(params, c_new, k_pe_new, s_new, in_dtype, positions, block_table, c_kv,
                                         k_pe, kv_scale, a);
  if (st != MLA_OK) return st;
  return launch_status(mla::launch_append(a, (hipStream_t)stream));
}

}  // extern "C"
