// C ABI of libmoe: argument validation, workspace layout and launch order.
// Nothing here computes; every step of the layer runs in the kernels of
// gate.hip, route.hip, expert.hip and combine.hip.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "moe_kernels.h"

using namespace moe;

// Scratch of moe_forward_static: one array per GPU, in the library's code
// object, held until the process ends.  Host code reaches it only through
// the device address hipGetSymbolAddress returns for the current device
// (scratch_ptr below); in host code the array's name is a stand-in, not a
// device address.
static __device__ __align__(256) unsigned char scratch[MOE_FORWARD_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status ok() {
  g_last_error.clear();
  return MOE_OK;
}

constexpr int MAX_K = 8;
constexpr int MAX_EXPERTS = 8192;  // route kernels keep 8 bytes per expert in LDS

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t elem_size(const moe_config* c) { return c->dtype == MOE_BF16 ? 2 : 4; }

// Every workspace region, at fixed offsets for a given configuration.
struct Layout {
  size_t idx, gate, thr, counts, offsets, perm, inv, bits, base, tiles, hid, ysorted, part,
      imp_part, imp, load;
  size_t idx_p, gate_p, counts_g, offsets_g, perm_g, inv_g, bits_g, base_g, tiles_g;
  size_t counts_u, offsets_u, perm_u, inv_u;
  size_t total;
  int nb, load_blocks;
};

Layout layout(const moe_config* c) {
  Layout L;
  const int64_t T = c->tokens, A = T * c->top_k;
  const int E = c->n_experts;
  L.nb = (int)((T + ROUTE_BLOCK_TOKENS - 1) / ROUTE_BLOCK_TOKENS);
  L.load_blocks = load_partial_blocks(T);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  L.idx = take(4 * (size_t)A);
  L.gate = take(4 * (size_t)A);
  L.thr = take(8 * (size_t)T);
  L.counts = take(4 * (size_t)E);
  L.offsets = take(4 * (size_t)(E + 1));
  L.perm = take(4 * (size_t)A);
  L.inv = take(4 * (size_t)A);
  L.bits = take(4 * (size_t)L.nb * E);
  L.base = take(4 * (size_t)L.nb * E);

  L.tiles = take(4 * (size_t)(E + 1));
  // the hidden layer in memory: only the unfused expert paths keep it there
  const bool fused_ffn = c->dtype == MOE_BF16 &&
                         fused_ffn_supported(c->d_model, c->d_hidden, c->ffn == MOE_FFN_SWIGLU);
  L.hid = take(fused_ffn ? 0 : elem_size(c) * (size_t)A * c->d_hidden);
  L.ysorted = take(elem_size(c) * (size_t)A * c->d_model);
  L.part = take(4 * (size_t)L.load_blocks * E);
  L.imp_part = take(gate_fuses_load(E) ? 4 * (size_t)L.nb * E : 0);
  L.imp = take(4 * (size_t)E);
  L.load = take(4 * (size_t)E);
  const int G = c->n_groups > 0 ? c->n_groups : 0;
  const int64_t Ag = T * (G ? c->k_groups : 0);
  L.idx_p = take(4 * (size_t)Ag);
  L.gate_p = take(4 * (size_t)Ag);
  L.counts_g = take(4 * (size_t)G);
  L.offsets_g = take(4 * (size_t)(G + 1));
  L.perm_g = take(4 * (size_t)Ag);
  L.inv_g = take(4 * (size_t)Ag);
  L.bits_g = take(4 * (size_t)L.nb * G);
  L.base_g = take(4 * (size_t)L.nb * G);
  L.tiles_g = take(4 * (size_t)(G + 1));
  // the routing without the capacity, for the balance statistics
  const bool cap = c->capacity > 0;
  L.counts_u = take(cap ? 4 * (size_t)E : 0);
  L.offsets_u = take(cap ? 4 * (size_t)(E + 1) : 0);
  L.perm_u = take(cap ? 4 * (size_t)A : 0);
  L.inv_u = take(cap ? 4 * (size_t)A : 0);
  L.total = o;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}

moe_status check_config(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (c->tokens < 0) return fail(MOE_ERR_INVALID_ARG, "tokens < 0");
  if (c->d_model < 1 || c->d_hidden < 1 || c->n_experts < 1)
    return fail(MOE_ERR_INVALID_ARG, "d_model, d_hidden and n_experts must be >= 1");
  if (c->top_k < 1 || c->top_k > c->n_experts)
    return fail(MOE_ERR_INVALID_ARG, "top_k must be in [1, n_experts]");
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", c->dtype);
  if (c->ffn != MOE_FFN_RELU && c->ffn != MOE_FFN_SWIGLU)
    return fail(MOE_ERR_INVALID_ARG, "unknown ffn %d", c->ffn);
  if (c->noisy != 0 && c->noisy != 1) return fail(MOE_ERR_INVALID_ARG, "noisy must be 0 or 1");
  if (c->capacity < 0) return fail(MOE_ERR_INVALID_ARG, "capacity < 0");
  if (c->n_groups < 0) return fail(MOE_ERR_INVALID_ARG, "n_groups < 0");
  if (c->n_groups > 0) {
    const int G = c->n_groups;
    if (c->n_experts % G != 0)
      return fail(MOE_ERR_INVALID_ARG, "n_experts %% n_groups != 0");
    if (c->k_groups < 1 || c->k_groups > G)
      return fail(MOE_ERR_INVALID_ARG, "k_groups must be in [1, n_groups]");
    if (c->k_per_group < 1 || c->k_per_group > c->n_experts / G)
      return fail(MOE_ERR_INVALID_ARG, "k_per_group must be in [1, n_experts / n_groups]");
    if (c->top_k != c->k_groups * c->k_per_group)
      return fail(MOE_ERR_INVALID_ARG, "top_k != k_groups * k_per_group");
  }
  if (c->top_k > MAX_K) return fail(MOE_ERR_UNSUPPORTED, "top_k > %d", MAX_K);
  if (c->n_experts > MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "n_experts > %d", MAX_EXPERTS);
  if (c->tokens * (int64_t)c->top_k > (int64_t)INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "tokens * top_k exceeds int32 positions");
  if (c->dtype == MOE_BF16 && (c->d_model % 64 != 0 || c->d_hidden % 64 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "bf16 needs d_model and d_hidden multiples of 64");
  return MOE_OK;
}

moe_status check_ws(const moe_config* c, void* ws, size_t ws_bytes) {
  const size_t need = layout(c).total;
  if (need == 0) return MOE_OK;
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  return MOE_OK;
}

// Packed gate geometry of cfg: table groups, experts per group, tables.
bool gate_packable(const moe_config* c) {
  return gate_pack_supported(c->dtype == MOE_BF16, c->d_model);
}
int gate_pack_groups(const moe_config* c) { return c->n_groups > 0 ? c->n_groups : 1; }
int gate_pack_tables(const moe_config* c) { return c->noisy ? 2 : 1; }

// The noise source of a kernel: the generator when the caller asks for it,
// else the caller's tensor (stream 1: the hierarchy's primary noise).
NoiseSrc noise_src(const moe_noise* n, const float* eps, int stream) {
  NoiseSrc s;
  if (n && n->in_kernel) {
    s.gen = 1;
    s.k0 = (uint32_t)(n->seed & 0xFFFFFFFFu);
    s.k1 = (uint32_t)(n->seed >> 32);
    s.stream = stream;
  } else {
    s.eps = eps;
  }
  return s;
}

bool has_noise(const moe_noise* n, const float* eps) { return (n && n->in_kernel) || eps; }

moe_status check_gate_inputs(const moe_config* c, const void* x, const moe_params* p,
                             const moe_noise* n) {
  if (!x && c->tokens > 0) return fail(MOE_ERR_INVALID_ARG, "x is NULL");
  if (!p) return fail(MOE_ERR_INVALID_ARG, "params is NULL");
  if (!p->w_gate) return fail(MOE_ERR_INVALID_ARG, "w_gate is NULL");
  // an empty batch reads no activations and no noise
  const bool rows = c->tokens > 0;
  if (c->noisy) {
    if (!n) return fail(MOE_ERR_INVALID_ARG, "noisy gate needs a moe_noise (noise is NULL)");
    if (rows && !has_noise(n, n ? n->eps : nullptr))
      return fail(MOE_ERR_INVALID_ARG, "noisy gate needs eps (or noise drawn in the kernels)");
    if (!p->w_noise) return fail(MOE_ERR_INVALID_ARG, "noisy gate needs w_noise");
  }
  if (p->w_gate_packed) {
    if (!gate_packable(c))
      return fail(MOE_ERR_UNSUPPORTED, "packed gate tables need bf16 and d_model %% 64 == 0");
    if (reinterpret_cast<uintptr_t>(p->w_gate_packed) & 15)
      return fail(MOE_ERR_INVALID_ARG, "w_gate_packed must be 16-byte aligned");
  }
  if (c->n_groups > 0) {
    if (!p->w_gate_p) return fail(MOE_ERR_INVALID_ARG, "hierarchy needs w_gate_p");
    if (p->bias) return fail(MOE_ERR_UNSUPPORTED, "bias is supported by the flat gate only");
    if (c->noisy && ((rows && !has_noise(n, n ? n->eps_p : nullptr)) || !p->w_noise_p))
      return fail(MOE_ERR_INVALID_ARG, "noisy hierarchy needs eps_p and w_noise_p");
  }
  return MOE_OK;
}

bool packable(const moe_config* c) {
  return c->dtype == MOE_BF16 && fused_ffn_supported(c->d_model, c->d_hidden, c->ffn);
}

moe_status check_expert_inputs(const moe_config* c, const moe_params* p) {
  if (!p) return fail(MOE_ERR_INVALID_ARG, "params is NULL");
  if (p->w_packed) {
    if (!packable(c)) return fail(MOE_ERR_UNSUPPORTED, "packed expert tables need bf16 ReLU, d_model 512");
    if (reinterpret_cast<uintptr_t>(p->w_packed) & 15)
      return fail(MOE_ERR_INVALID_ARG, "w_packed must be 16-byte aligned");
    return MOE_OK;
  }
  if (!p->w1 || !p->w2) return fail(MOE_ERR_INVALID_ARG, "w1 / w2 is NULL");
  if (c->ffn == MOE_FFN_SWIGLU && !p->w3) return fail(MOE_ERR_INVALID_ARG, "SwiGLU needs w3");
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

#define MOE_TRY(expr)              \
  do {                             \
    moe_status _st = (expr);       \
    if (_st != MOE_OK) return _st; \
  } while (0)

// ---- enqueue helpers (arguments already validated) -------------------------

// part != null (flat noisy gate with E <= GATE_FUSED_LOAD_MAX_E): the gate
// kernel also writes the smooth-load partial sums.  bits != null (flat gate):
// it also writes the routing masks of its 32-token tiles.
moe_status do_gate(const moe_config* c, const Layout& L, const void* x, const moe_params* p,
                   const moe_noise* n, int32_t* idx, float* gate, float* thr, float* part,
                   uint32_t* bits, float* imp_part, void* ws, hipStream_t s) {
  const bool bf16 = c->dtype == MOE_BF16;
  const bool noisy = c->noisy != 0;
  if (c->n_groups == 0) {
    GateFlatArgs a;
    a.x = x;
    a.w_gate = p->w_gate;
    a.w_noise = noisy ? p->w_noise : nullptr;
    a.bias = p->bias;
    a.noise = noisy ? noise_src(n, n ? n->eps : nullptr, 0) : NoiseSrc();
    a.T = c->tokens;
    a.d = c->d_model;
    a.E = c->n_experts;
    a.k = c->top_k;
    a.idx = idx;
    a.gate = gate;
    a.thr = thr;
    a.part = part;
    a.bits = bits;
    a.imp_part = imp_part;
    a.w_pack = p->w_gate_packed;
    a.pack_nt = gate_pack_tables(c);
    return hip_status(launch_gate_flat(a, bf16, s), "gate");
  }
  const int G = c->n_groups, kg = c->k_groups;
  int32_t* idx_p = at<int32_t>(ws, L.idx_p);
  float* gate_p = at<float>(ws, L.gate_p);
  GateFlatArgs a;
  a.x = x;
  a.w_gate = p->w_gate_p;
  a.w_noise = noisy ? p->w_noise_p : nullptr;
  a.bias = nullptr;
  a.noise = noisy ? noise_src(n, n ? n->eps_p : nullptr, 1) : NoiseSrc();
  a.T = c->tokens;
  a.d = c->d_model;
  a.E = G;
  a.k = kg;
  a.idx = idx_p;
  a.gate = gate_p;
  a.thr = nullptr;
  a.part = nullptr;
  a.bits = nullptr;
  MOE_TRY(hip_status(launch_gate_flat(a, bf16, s), "primary gate"));
  if (c->tokens == 0) return MOE_OK;
  RouteArgs r;
  r.idx = idx_p;
  r.T = c->tokens;
  r.k = kg;
  r.E = G;
  r.NB = L.nb;
  r.bits = at<uint32_t>(ws, L.bits_g);
  r.base = at<int32_t>(ws, L.base_g);
  r.have_bits = 0;
  r.counts = at<int32_t>(ws, L.counts_g);
  r.offsets = at<int32_t>(ws, L.offsets_g);
  r.perm = at<int32_t>(ws, L.perm_g);
  r.inv = at<int32_t>(ws, L.inv_g);
  int32_t* tiles_g = at<int32_t>(ws, L.tiles_g);
  // the secondary gate's row tiles (64 rows once the groups average as many:
  // each table fragment fetched from L2 then serves twice the rows)
  const int grows = gate_group_tile_rows(c->dtype == MOE_BF16, c->d_model, c->tokens * kg, G);
  r.tile_rows = grows;
  r.tiles = tiles_g;
  r.desc = nullptr;
  MOE_TRY(hip_status(launch_route(r, s), "group routing"));
  GateGroupArgs ga;
  ga.x = x;
  ga.w_gate = p->w_gate;
  ga.w_noise = noisy ? p->w_noise : nullptr;
  ga.noise = noisy ? noise_src(n, n ? n->eps : nullptr, 0) : NoiseSrc();
  ga.d = c->d_model;
  ga.G = G;
  ga.Eg = c->n_experts / G;
  ga.kg = kg;
  ga.kpg = c->k_per_group;
  ga.perm_g = r.perm;
  ga.offsets_g = r.offsets;
  ga.tiles_g = tiles_g;
  ga.gate_p = gate_p;
  ga.idx = idx;
  ga.gate = gate;
  ga.w_pack = p->w_gate_packed;
  ga.pack_nt = gate_pack_tables(c);
  ga.tile_rows = grows;
  const int64_t grid = (c->tokens * kg + grows - 1) / grows + G;
  return hip_status(launch_gate_group(ga, (int)grid, bf16, s), "secondary gate");
}

// Expert-stage tile rows of this configuration (0: no tile map needed).
int expert_tile_rows(const moe_config* c) {
  if (c->dtype != MOE_BF16) return 0;
  return ffn_tile_rows(true, c->d_model, c->d_hidden, c->ffn == MOE_FFN_SWIGLU,
                       c->tokens * c->top_k, c->n_experts);
}

// have_bits: the flat gate already wrote the routing masks.  with_tiles: also
// build the expert stage's tile map.
// Balance statistics reduced by the routing step (flat gate with per-tile
// partials); imp_part null: none.
struct RouteStats {
  const float* imp_part = nullptr;
  const float* load_part = nullptr;
  float *importance = nullptr, *load = nullptr, *out = nullptr;
  float w_imp = 0.f, w_load = 0.f;
};

moe_status do_route(const moe_config* c, const Layout& L, const int32_t* idx, int32_t* counts,
                    int32_t* offsets, int32_t* perm, int32_t* inv, bool have_bits,
                    bool with_tiles, void* ws, hipStream_t s, const RouteStats& st = RouteStats(),
                    bool capped = true) {
  RouteArgs r;
  r.capacity = capped ? c->capacity : 0;
  r.idx = idx;
  r.T = c->tokens;
  r.k = c->top_k;
  r.E = c->n_experts;
  r.NB = L.nb;
  r.bits = at<uint32_t>(ws, L.bits);
  r.base = at<int32_t>(ws, L.base);
  r.have_bits = have_bits ? 1 : 0;
  r.counts = counts;
  r.offsets = offsets;
  r.perm = perm;
  r.inv = inv;
  r.tile_rows = with_tiles ? expert_tile_rows(c) : 0;
  r.tiles = at<int32_t>(ws, L.tiles);
  r.desc = nullptr;
  if (st.imp_part) {
    r.imp_part = st.imp_part;
    r.load_part = st.load_part;
    r.importance = st.importance;
    r.load = st.load;
    r.bal_out = st.out;
    r.w_imp = st.w_imp;
    r.w_load = st.w_load;
  }
  return hip_status(launch_route(r, s), "route");
}

// tiles_ready: the routing step already built the tile map.
moe_status do_ffn(const moe_config* c, const Layout& L, const void* x, const int32_t* perm,
                  const int32_t* offsets, const moe_params* p, void* y_sorted, bool tiles_ready,
                  void* ws, hipStream_t s) {
  const bool bf16 = c->dtype == MOE_BF16;
  const int sw = c->ffn == MOE_FFN_SWIGLU;
  FfnArgs f;
  f.x = x;
  f.perm = perm;
  f.k = c->top_k;
  f.offsets = offsets;
  int32_t* tiles = at<int32_t>(ws, L.tiles);
  f.tiles = tiles;
  f.E = c->n_experts;
  f.d = c->d_model;
  f.h = c->d_hidden;
  f.w1 = p->w1;
  f.w3 = sw ? p->w3 : nullptr;
  f.w2 = p->w2;
  f.hid = at<void>(ws, L.hid);
  f.y_sorted = y_sorted;
  f.A = c->tokens * c->top_k;
  f.wpacked = p->w_packed;
  if (f.A == 0) return MOE_OK;
  const int rows = bf16 ? ffn_tile_rows(bf16, c->d_model, c->d_hidden, sw, f.A, c->n_experts) : 0;
  if (rows > 0 && !tiles_ready)
    MOE_TRY(hip_status(launch_tile_map(offsets, c->n_experts, rows, tiles, nullptr, s),
                       "expert tiles"));
  return hip_status(launch_expert_ffn(f, bf16, sw, s), "experts");
}

// The smooth load's partial sums (flat noisy gate), recomputing the
// projections from the gate's thresholds.
moe_status smooth_load_partials(const moe_config* c, const Layout& L, const void* x,
                                const moe_params* p, const int32_t* idx, const float* thr,
                                void* ws, hipStream_t s) {
  LoadArgs la;
  la.x = x;
  la.w_gate = p->w_gate;
  la.w_noise = p->w_noise;
  la.bias = p->bias;
  la.idx = idx;
  la.thr = thr;
  la.T = c->tokens;
  la.d = c->d_model;
  la.E = c->n_experts;
  la.k = c->top_k;
  la.part = at<float>(ws, L.part);
  la.w_pack = p->w_gate_packed;
  return hip_status(launch_load_partial(la, c->dtype == MOE_BF16, s), "load");
}

// have_part: the smooth-load partial sums are already written (by the gate
// kernel, or by smooth_load_partials on the stream s follows).
moe_status do_balance(const moe_config* c, const Layout& L, const void* x, const moe_params* p,
                      const int32_t* idx, const float* gate, const float* thr,
                      const int32_t* perm, const int32_t* offsets, float wi, float wl,
                      float* importance, float* load, float* out, bool have_part, void* ws,
                      hipStream_t s) {
  const int E = c->n_experts;
  const bool smooth = c->n_groups == 0 && c->noisy && c->tokens > 0;
  float* part = smooth ? at<float>(ws, L.part) : nullptr;
  if (smooth && !have_part) MOE_TRY(smooth_load_partials(c, L, x, p, idx, thr, ws, s));
  BalanceArgs b;
  b.perm = perm;
  b.offsets = offsets;
  b.gate = gate;
  b.part = part;
  b.blocks = L.load_blocks;
  b.E = E;
  b.k = c->top_k;
  b.w_imp = wi;
  b.w_load = wl;
  b.importance = importance;
  b.load = load;
  b.out = out;
  return hip_status(launch_balance(b, s), "balance");
}


// ---- backward layout and launch order ----------------------------------------

struct BwLayout {
  size_t dimp, dload, dhk, rinfo, dclean, draw, dbias_part, dxg, tiles, tiles_big, zero, hid, dp, db, dxs, part_g,
      part_n, xs, dys;
  // hierarchy: per-slot and per-group score gradients, and the routing
  // without capacity (when the forward capped it) for the secondary tables
  size_t cs, ns, dcp, drp, r_bits, r_base, r_counts, r_offsets, r_perm, r_inv;
  // flat bf16 gate with E <= 256: the gate tables transposed for the fused dx product
  size_t wgt, wnt;
  int e16;
  size_t total;
  int nblk, nchunk, nb;
  int64_t kchunk;
};

BwLayout bw_layout(const moe_config* c) {
  BwLayout L;
  const int64_t T = c->tokens, A = T * c->top_k;
  const int E = c->n_experts, d = c->d_model, h = c->d_hidden;
  const size_t es = elem_size(c);
  const bool sw = c->ffn == MOE_FFN_SWIGLU;
  const bool hier = c->n_groups > 0;
  const int G = hier ? c->n_groups : 0;
  // rows of the dense gate-table products: the experts, or the hierarchy's groups
  const int Etab = hier ? G : E;
  L.nblk = (int)((T + 31) / 32);
  L.nb = (int)((T + ROUTE_BLOCK_TOKENS - 1) / ROUTE_BLOCK_TOKENS);
  // gate-table products: K = tokens split into chunks, enough workgroups
  const int64_t tiles_mn = ((Etab + 127) / 128) * (int64_t)((d + 127) / 128);
  int64_t nch = (1024 + tiles_mn - 1) / tiles_mn;
  // chunks of at least 256 tokens (bf16, 64-wide K slices) or 64 (fp32,
  // 16-wide slices)
  const int64_t min_chunk = es == 2 ? 256 : 64;
  nch = std::min<int64_t>(nch, std::max<int64_t>(1, (T + min_chunk - 1) / min_chunk));
  nch = std::max<int64_t>(nch, 1);
  int64_t kc = (T + nch - 1) / nch;
  kc = std::max<int64_t>(32, (kc + 31) / 32 * 32);
  L.kchunk = kc;
  L.nchunk = (int)std::max<int64_t>(1, (T + kc - 1) / kc);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  const bool flat = !hier;
  L.dimp = take(4 * (size_t)E);
  L.dload = take(4 * (size_t)E);
  L.dhk = take(flat ? 4 * (size_t)A : 0);
  L.rinfo = take(flat ? 16 * (size_t)T : 0);
  L.dclean = take(flat ? 4 * (size_t)T * E : 0);
  L.draw = take(flat && c->noisy ? 4 * (size_t)T * E : 0);
  L.dbias_part = take(flat ? 4 * (size_t)L.nblk * E : 0);
  L.cs = take(hier ? 4 * (size_t)A : 0);
  L.ns = take(hier && c->noisy ? 4 * (size_t)A : 0);
  L.dcp = take(hier ? 4 * (size_t)T * G : 0);
  L.drp = take(hier && c->noisy ? 4 * (size_t)T * G : 0);
  const bool reroute = hier && c->capacity > 0;
  L.r_bits = take(reroute ? 4 * (size_t)L.nb * E : 0);
  L.r_base = take(reroute ? 4 * (size_t)L.nb * E : 0);
  L.r_counts = take(reroute ? 4 * (size_t)E : 0);
  L.r_offsets = take(reroute ? 4 * (size_t)(E + 1) : 0);
  L.r_perm = take(reroute ? 4 * (size_t)A : 0);
  L.r_inv = take(reroute ? 4 * (size_t)A : 0);
  const bool fused_dxg = flat && es == 2 && E <= bw_fused_dxg_max_experts();
  L.e16 = fused_dxg ? (E + 15) / 16 * 16 : 0;
  L.wgt = take(fused_dxg ? 2 * (size_t)d * L.e16 : 0);
  L.wnt = take(fused_dxg && c->noisy ? 2 * (size_t)d * L.e16 : 0);
  L.dxg = take(4 * (size_t)T * d);
  L.tiles = take(4 * (size_t)(E + 1));
  L.tiles_big = take(4 * (size_t)(E + 1));
  L.zero = take(2 * (size_t)std::max(std::max(h, d), 128));
  L.hid = take(es * (size_t)A * h);
  L.dp = take(es * (size_t)A * h);
  L.db = take(sw ? es * (size_t)A * h : 0);
  L.dxs = take(es * (size_t)A * d);
  L.part_g = take(4 * (size_t)L.nchunk * Etab * d);
  L.part_n = take(c->noisy ? 4 * (size_t)L.nchunk * Etab * d : 0);
  L.xs = take(es * (size_t)A * d);
  L.dys = take(es * (size_t)A * d);
  L.total = o;
  return L;
}

// Operands: rows (element (r, k) at r*ld + k) or columns (at k*ld + r).
BwOp op_rows(const void* ptr, int64_t ld, bool f32) {
  BwOp o;
  o.p = ptr;
  o.ld = ld;
  o.kind = f32 ? BW_KF : BW_KB;
  return o;
}

BwOp op_cols(const void* ptr, int64_t ld, bool f32) {
  BwOp o = op_rows(ptr, ld, f32);
  o.kind = f32 ? BW_TF : BW_TB;
  return o;
}

BwOp per_expert(BwOp o, int64_t estride) {
  o.estride = estride;
  return o;
}

BwOp low_half(BwOp o) {
  o.lo = 1;
  return o;
}

// a product with one operand pair; add_pair appends pairs summed into it
BwGemm product(const BwOp& a, const BwOp& b) {
  BwGemm q;
  q.a[0] = a;
  q.b[0] = b;
  q.npair = 1;
  return q;
}

void add_pair(BwGemm& q, const BwOp& a, const BwOp& b) {
  q.a[q.npair] = a;
  q.b[q.npair] = b;
  ++q.npair;
}

// A gate table's gradient: out[rows][d] = coef^T x for coef [T][rows] fp32,
// the tokens split into chunks whose partial products are summed in order.
moe_status gate_table_grad(const moe_config* c, const BwLayout& L, const void* x,
                           const float* coef, int rows, void* out, float* part, hipStream_t s) {
  if (!out) return MOE_OK;
  const bool bf16 = c->dtype == MOE_BF16;
  const bool f32 = !bf16;
  const int d = c->d_model;
  BwGemm q = product(op_cols(coef, rows, true), op_cols(x, d, f32));
  q.mode = BW_PLAIN;
  // bf16 products carry the fp32 score gradients as hi + lo halves
  if (bf16) add_pair(q, low_half(q.a[0]), q.b[0]);
  q.M = rows;
  q.N = d;
  q.K = c->tokens;
  q.kchunk = L.kchunk;
  q.C = part;
  q.c_f32 = 1;
  q.ldc = d;
  q.c_chunk = (int64_t)rows * d;
  const int64_t grid = (int64_t)L.nchunk * ((rows + 127) / 128) * ((d + 127) / 128);
  MOE_TRY(hip_status(launch_bw_gemm(q, bf16, grid, s), "backward gate tables"));
  return hip_status(launch_bw_sum_chunks(part, L.nchunk, (int64_t)rows * d, bf16, out, s),
                    "backward gate table sum");
}

// The same for bf16 coefficients already split into hi and lo halves [T][rows].
// zero: a row of at least 128 zeros (bf16), read past the last token
moe_status gate_table_grad_halves(const moe_config* c, const BwLayout& L, const void* x,
                                  const bf16_t* hi, const bf16_t* lo, int rows, void* out,
                                  float* part, const void* zero, hipStream_t s) {
  if (!out) return MOE_OK;
  const int d = c->d_model;
  BwGemm q = product(op_cols(hi, rows, false), op_cols(x, d, false));
  q.mode = BW_PLAIN;
  add_pair(q, op_cols(lo, rows, false), q.b[0]);
  q.M = rows;
  q.N = d;
  q.K = c->tokens;
  q.kchunk = L.kchunk;
  q.C = part;
  q.c_f32 = 1;
  q.ldc = d;
  q.c_chunk = (int64_t)rows * d;
  q.zero = zero;
  const int64_t grid = (int64_t)L.nchunk * ((rows + 127) / 128) * ((d + 127) / 128);
  MOE_TRY(hip_status(launch_bw_gemm(q, true, grid, s), "backward gate tables"));
  return hip_status(launch_bw_sum_chunks(part, L.nchunk, (int64_t)rows * d, true, out, s),
                    "backward gate table sum");
}

// The hierarchy's gate side: score gradients of both levels and dx's share
// (one wave per token), the primary tables as dense products over tokens,
// the secondary tables as per-expert sums over the routed rows of the
// gate's choice (rerouted without the capacity when the forward dropped).
moe_status hier_gate_backward(const moe_config* c, const BwLayout& L, const void* x,
                              const moe_params* p, const moe_noise* n, const moe_saved* sv,
                              const void* dy, const float* dimp, moe_grads* g, void* ws,
                              hipStream_t s) {
  const int64_t T = c->tokens;
  const int E = c->n_experts, d = c->d_model, k = c->top_k, G = c->n_groups;
  const bool bf16 = c->dtype == MOE_BF16;
  const bool noisy = c->noisy != 0;
  float* cs = at<float>(ws, L.cs);
  float* ns = noisy ? at<float>(ws, L.ns) : nullptr;
  float* dcp = at<float>(ws, L.dcp);
  float* drp = noisy ? at<float>(ws, L.drp) : nullptr;
  if (T > 0) {
    BwHierGateArgs a;
    a.y_sorted = sv->y_sorted;
    a.inv = sv->inv;
    a.idx = sv->topk_idx;
    a.gate = sv->topk_gate;
    a.dy = dy;
    a.dimp = dimp;
    a.x = x;
    a.w_gate = p->w_gate;
    a.w_noise = noisy ? p->w_noise : nullptr;
    a.w_gate_p = p->w_gate_p;
    a.w_noise_p = noisy ? p->w_noise_p : nullptr;
    a.noise = noisy ? noise_src(n, n ? n->eps : nullptr, 0) : NoiseSrc();
    a.noise_p = noisy ? noise_src(n, n ? n->eps_p : nullptr, 1) : NoiseSrc();
    a.T = T;
    a.k = k;
    a.d = d;
    a.G = G;
    a.Eg = E / G;
    a.kpg = c->k_per_group;
    a.dxg = at<float>(ws, L.dxg);
    a.cs = cs;
    a.ns = ns;
    a.dcp = dcp;
    a.drp = drp;
    MOE_TRY(hip_status(launch_bw_hier_gate(a, bf16, s), "backward hierarchy gate"));
  }
  MOE_TRY(gate_table_grad(c, L, x, dcp, G, g->dw_gate_p, at<float>(ws, L.part_g), s));
  if (noisy)
    MOE_TRY(gate_table_grad(c, L, x, drp, G, g->dw_noise_p, at<float>(ws, L.part_n), s));
  if (!g->dw_gate && !g->dw_noise) return MOE_OK;
  const int32_t* offsets = sv->offsets;
  const int32_t* perm = sv->perm;
  if (c->capacity > 0 && T > 0) {
    Layout R{};
    R.nb = L.nb;
    R.bits = L.r_bits;
    R.base = L.r_base;
    R.tiles = L.r_counts;  // no tile map is built (with_tiles false)
    int32_t* offs = at<int32_t>(ws, L.r_offsets);
    int32_t* pm = at<int32_t>(ws, L.r_perm);
    MOE_TRY(do_route(c, R, sv->topk_idx, at<int32_t>(ws, L.r_counts), offs, pm,
                     at<int32_t>(ws, L.r_inv), false, false, ws, s, RouteStats(), false));
    offsets = offs;
    perm = pm;
  }
  BwRowSumArgs r;
  r.x = x;
  r.perm = perm;
  r.offsets = offsets;
  r.k = k;
  r.E = E;
  r.d = d;
  const bool both = g->dw_gate && g->dw_noise;
  r.c0 = g->dw_gate ? cs : ns;
  r.out0 = g->dw_gate ? g->dw_gate : g->dw_noise;
  r.c1 = both ? ns : nullptr;
  r.out1 = both ? g->dw_noise : nullptr;
  return hip_status(launch_bw_expert_rowsum(r, bf16, s), "backward hierarchy tables");
}

// A second stream per device for the backward's expert side: created on the
// device's first backward call and kept until the process ends, at the
// default priority.  Backward calls on one device share it, so their expert
// sides run one after another.
constexpr int SIDE_MAX_DEVICES = 64;
std::mutex g_side_mutex;
hipStream_t g_side_stream[SIDE_MAX_DEVICES];

moe_status side_stream(hipStream_t* out) {
  *out = nullptr;
  int dev = -1;
  MOE_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= SIDE_MAX_DEVICES) return MOE_OK;  // one stream, then
  std::lock_guard<std::mutex> lock(g_side_mutex);
  if (!g_side_stream[dev])
    MOE_TRY(hip_status(hipStreamCreateWithFlags(&g_side_stream[dev], hipStreamNonBlocking),
                       "hipStreamCreateWithFlags"));
  *out = g_side_stream[dev];
  return MOE_OK;
}

// The fork of the caller's stream onto the side stream, and the join back.
// The caller's stream waits for the join on every return path, so that work
// queued on it after a failed call still follows everything the call launched.
struct SideJoin {
  hipStream_t main, side;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr, ev_mid = nullptr;
  bool forked = false, recorded = false, waited = false;
  explicit SideJoin(hipStream_t s) : main(s), side(s) {}
  SideJoin(const SideJoin&) = delete;
  SideJoin& operator=(const SideJoin&) = delete;
  moe_status fork() {
    hipStream_t t = nullptr;
    MOE_TRY(side_stream(&t));
    if (!t || t == main) return MOE_OK;
    MOE_TRY(hip_status(hipEventCreateWithFlags(&ev_fork, hipEventDisableTiming), "hipEventCreate"));
    MOE_TRY(hip_status(hipEventCreateWithFlags(&ev_join, hipEventDisableTiming), "hipEventCreate"));
    MOE_TRY(hip_status(hipEventRecord(ev_fork, main), "hipEventRecord"));
    MOE_TRY(hip_status(hipStreamWaitEvent(t, ev_fork, 0), "hipStreamWaitEvent"));
    side = t;
    forked = true;
    return MOE_OK;
  }
  // the side stream waits for everything queued on the caller's stream so far
  moe_status side_follows_main() {
    if (!forked) return MOE_OK;
    if (!ev_mid)
      MOE_TRY(hip_status(hipEventCreateWithFlags(&ev_mid, hipEventDisableTiming), "hipEventCreate"));
    MOE_TRY(hip_status(hipEventRecord(ev_mid, main), "hipEventRecord"));
    return hip_status(hipStreamWaitEvent(side, ev_mid, 0), "hipStreamWaitEvent");
  }
  moe_status record() {
    if (!forked || recorded) return MOE_OK;
    MOE_TRY(hip_status(hipEventRecord(ev_join, side), "hipEventRecord"));
    recorded = true;
    return MOE_OK;
  }
  moe_status wait() {
    if (!forked || waited) return MOE_OK;
    MOE_TRY(record());
    waited = true;
    return hip_status(hipStreamWaitEvent(main, ev_join, 0), "hipStreamWaitEvent");
  }
  ~SideJoin() {
    if (forked && !waited) {
      if (!recorded) (void)hipEventRecord(ev_join, side);
      (void)hipStreamWaitEvent(main, ev_join, 0);
    }
    if (ev_fork) (void)hipEventDestroy(ev_fork);
    if (ev_join) (void)hipEventDestroy(ev_join);
    if (ev_mid) (void)hipEventDestroy(ev_mid);
  }
};

moe_status do_backward(const moe_config* c, const BwLayout& L, const void* x, const moe_params* p,
                       const moe_noise* n, const moe_saved* sv, const void* dy, float wi,
                       float wl, moe_grads* g, void* ws, hipStream_t s) {
  const int64_t T = c->tokens, A = T * c->top_k;
  const int E = c->n_experts, d = c->d_model, h = c->d_hidden, k = c->top_k;
  const bool bf16 = c->dtype == MOE_BF16;
  const bool f32 = !bf16;
  const bool noisy = c->noisy != 0;
  const bool sw = c->ffn == MOE_FFN_SWIGLU;
  float* dimp = at<float>(ws, L.dimp);
  float* dload = at<float>(ws, L.dload);
  // 5. experts
  void* hid = at<void>(ws, L.hid);
  void* dp = at<void>(ws, L.dp);
  void* db = sw ? at<void>(ws, L.db) : nullptr;
  void* dxs = at<void>(ws, L.dxs);
  const int64_t hd = (int64_t)h * d;
  // The expert side shares no buffer with the gate side (1-4) up to the dx
  // assembly, so it runs on a second stream of the device (see side_stream)
  // while the gate side runs on the caller's.
  auto expert_side = [&](hipStream_t se) -> moe_status {
    // the routed rows of x and the gate-scaled output gradients, in expert order
    void* xs = at<void>(ws, L.xs);
    void* dys = at<void>(ws, L.dys);
    // the fused hidden-layer kernel gathers the rows itself
    const bool gathers_in_kernel =
        !bw_hidden_big_tiles(bf16, A, E) && bw_hidden_fused_supported(bf16, d, h, sw);
    if (A > 0 && !gathers_in_kernel) {
      MOE_TRY(hip_status(launch_bw_gather_rows(x, sv->perm, k, nullptr, A, d, bf16, xs, se),
                         "backward gather x"));
      MOE_TRY(hip_status(launch_bw_gather_rows(dy, sv->perm, k, sv->topk_gate, A, d, bf16, dys, se),
                         "backward gather dy"));
    }
    // experts averaging >= 256 rows (bf16): the large-tile products
    const bool big = bw_hidden_big_tiles(bf16, A, E);
    if (A > 0) {
      int32_t* tiles = at<int32_t>(ws, L.tiles);
      // rows per tile of the row-position products: 32 when the experts
      // average at most 32 rows (a quarter of the accumulators; three
      // workgroups per compute unit keep more table loads in flight)
      const int prow = bw_pos_tile_rows(bf16, A, E);
      // ReLU at d_model 512: the hidden layer and dX on per-tile streaming
      // kernels, which find their tiles from the offsets
      const bool fz = !big && bw_hidden_fused_supported(bf16, d, h, sw);
      if (!fz)
        MOE_TRY(hip_status(launch_tile_map(sv->offsets, E, prow, tiles, nullptr, se),
                           "backward tiles"));
      const int64_t row_tiles = (A + prow - 1) / prow + E;
      int32_t* tiles_big = at<int32_t>(ws, L.tiles_big);
      // dX on the large tiles from 128 rows per expert on average: one 256-row
      // tile then holds most experts whole, so each of an expert's two column
      // tiles reads its dP rows once (flat256 backward 0.849 -> 0.833 ms)
      const bool big_dx = bf16 && A >= 128 * (int64_t)E;
      if (big || (big_dx && !fz))
        MOE_TRY(hip_status(launch_tile_map(sv->offsets, E, bw_hidden_big_rows(), tiles_big,
                                           nullptr, se),
                           "backward tiles"));
      if (big) {
        // large experts, on the forward's large-tile GEMM: dHid = dY W2 into
        // the dP (dA) buffer, then the hidden layer recomputed with the
        // activation's derivative applied in the epilogue
        BwBigProduct q;
        q.a = dys;
        q.a2 = nullptr;
        q.b = p->w2;
        q.b2 = nullptr;
        q.A = A;
        q.E = E;
        q.N = h;
        q.K = d;
        q.offsets = sv->offsets;
        q.tiles = tiles_big;
        q.c = dp;
        MOE_TRY(hip_status(launch_bw_big_product(q, se), "backward dhid"));
        BwHiddenArgs ha;
        ha.xs = xs;
        ha.offsets = sv->offsets;
        ha.tiles = tiles_big;
        ha.E = E;
        ha.d = d;
        ha.h = h;
        ha.A = A;
        ha.w1 = p->w1;
        ha.w3 = sw ? p->w3 : nullptr;
        ha.hid = hid;
        ha.d1 = dp;
        ha.d3 = db;
        MOE_TRY(hip_status(launch_bw_hidden_big(ha, sw, se), "backward hidden"));
      } else if (fz) {
        // the hidden layer recomputed with its gradient, each tile streaming
        // W1 and then W2 once
        BwHidFusedArgs ha;
        ha.x = x;
        ha.dy = dy;
        ha.perm = sv->perm;
        ha.gate = sv->topk_gate;
        ha.k = k;
        ha.xs = xs;
        ha.dys = dys;
        ha.offsets = sv->offsets;
        ha.E = E;
        ha.h = h;
        ha.w1 = p->w1;
        ha.w2 = p->w2;
        ha.wp = p->w_packed;
        ha.hid = hid;
        ha.dp = dp;
        MOE_TRY(hip_status(launch_bw_hidden_fused(ha, A, se), "backward hidden"));
      } else {
        // hidden layer recomputed with its gradient
        BwGemm q = product(op_rows(xs, d, f32), per_expert(op_rows(p->w1, d, f32), hd));
        q.mode = BW_POS;
        q.epi = sw ? BW_EPI_SWIGLU : BW_EPI_RELU;
        q.a[1] = op_rows(dys, d, f32);
        q.b[1] = per_expert(op_cols(p->w2, h, f32), hd);
        if (sw) q.b[2] = per_expert(op_rows(p->w3, d, f32), hd);
        q.M = A;
        q.N = h;
        q.K = d;
        q.offsets = sv->offsets;
        q.tiles = tiles;
        q.pos_rows = prow;
        q.E = E;
        q.C = hid;
        q.C2 = dp;
        q.C3 = db;
        MOE_TRY(hip_status(launch_bw_gemm(q, bf16, row_tiles * ((h + 127) / 128), se),
                           "backward hidden"));
      }
      // dX = dP W1 (+ dB W3), per routed row
      if (fz) {
        BwDxFusedArgs da;
        da.dp = dp;
        da.offsets = sv->offsets;
        da.E = E;
        da.h = h;
        da.w1 = p->w1;
        da.dxs = dxs;
        MOE_TRY(hip_status(launch_bw_dx_fused(da, A, se), "backward expert dx"));
      } else if (big || big_dx) {
        BwBigProduct q;
        q.a = dp;
        q.a2 = sw ? db : nullptr;
        q.b = p->w1;
        q.b2 = sw ? p->w3 : nullptr;
        q.A = A;
        q.E = E;
        q.N = d;
        q.K = h;
        q.offsets = sv->offsets;
        q.tiles = tiles_big;
        q.c = dxs;
        MOE_TRY(hip_status(launch_bw_big_product(q, se), "backward expert dx"));
      } else {
        BwGemm r = product(op_rows(dp, h, f32), per_expert(op_cols(p->w1, d, f32), hd));
        r.mode = BW_POS;
        if (sw) add_pair(r, op_rows(db, h, f32), per_expert(op_cols(p->w3, d, f32), hd));
        r.M = A;
        r.N = d;
        r.K = h;
        r.offsets = sv->offsets;
        r.tiles = tiles;
        r.pos_rows = prow;
        r.E = E;
        r.C = dxs;
        r.c_f32 = f32 ? 1 : 0;  // in the layer dtype, like the expert outputs
        r.ldc = d;
        MOE_TRY(hip_status(launch_bw_gemm(r, bf16, row_tiles * ((d + 127) / 128), se),
                           "backward expert dx"));
      }
    }
    // positions past an expert's rows (and, in the products that load
    // straight into LDS, rows past a tile) are read from a row of zeros,
    // filled before the fork
    void* zero = at<void>(ws, L.zero);
    // table gradients, one problem per expert over its rows (zero without rows)
    auto wgrad = [&](void* out, BwOp a, BwOp b, int64_t M, int64_t N, const char* what) {
      if (!out) return MOE_OK;
      BwGemm q = product(a, b);
      q.mode = BW_WGT;
      q.M = M;
      q.N = N;
      q.offsets = sv->offsets;
      q.E = E;
      q.C = out;
      q.c_f32 = f32 ? 1 : 0;
      q.ldc = N;
      q.c_estride = M * N;
      q.zero = bf16 ? zero : nullptr;
      const int64_t grid = (int64_t)E * ((M + 127) / 128) * ((N + 127) / 128);
      return hip_status(launch_bw_gemm(q, bf16, grid, se), what);
    };
    if (big) {
      auto wgrad_big = [&](void* out, const void* a, int M, const void* b, int N,
                           const char* what) {
        if (!out) return MOE_OK;
        BwBigWgrad q;
        q.a = a;
        q.b = b;
        q.E = E;
        q.M = M;
        q.N = N;
        q.offsets = sv->offsets;
        q.zero = zero;
        q.c = out;
        return hip_status(launch_bw_big_wgrad(q, se), what);
      };
      MOE_TRY(wgrad_big(g->dw1, dp, h, xs, d, "backward dw1"));
      if (sw) MOE_TRY(wgrad_big(g->dw3, db, h, xs, d, "backward dw3"));
      MOE_TRY(wgrad_big(g->dw2, dys, d, hid, h, "backward dw2"));
    } else {
      MOE_TRY(wgrad(g->dw1, op_cols(dp, h, f32), op_cols(xs, d, f32), h, d, "backward dw1"));
      if (sw)
        MOE_TRY(wgrad(g->dw3, op_cols(db, h, f32), op_cols(xs, d, f32), h, d, "backward dw3"));
      MOE_TRY(wgrad(g->dw2, op_cols(dys, d, f32), op_cols(hid, h, f32), d, h, "backward dw2"));
    }
    return MOE_OK;
  };
  if (bf16)
    MOE_TRY(hip_status(launch_fill_i32(at<int32_t>(ws, L.zero),
                                       std::max(std::max(h, d), 128) / 2, 0, s),
                       "backward zero row"));
  SideJoin join(s);
  MOE_TRY(join.fork());
  MOE_TRY(expert_side(join.side));
  MOE_TRY(join.record());
  // 1. CV^2 gradients of the two balance losses
  const bool use_imp = wi != 0.f && T > 0;
  const bool smooth = noisy && wl != 0.f && T > 0;
  MOE_TRY(hip_status(launch_bw_cv2_grad(use_imp ? sv->importance : nullptr,
                                        smooth ? sv->load : nullptr, E, wi, wl, dimp, dload, s),
                     "backward cv2"));
  float* dxg = at<float>(ws, L.dxg);
  if (c->n_groups > 0) {
    MOE_TRY(hier_gate_backward(c, L, x, p, n, sv, dy, use_imp ? dimp : nullptr, g, ws, s));
  } else {
  // 2. kept-gate gradients through the combine and the importance loss
  float* dhk = at<float>(ws, L.dhk);
  if (T > 0) {
    BwGateOutArgs go;
    go.y_sorted = sv->y_sorted;
    go.inv = sv->inv;
    go.idx = sv->topk_idx;
    go.gate = sv->topk_gate;
    go.dy = dy;
    go.dimp = use_imp ? dimp : nullptr;
    go.T = T;
    go.k = k;
    go.d = d;
    go.dhk = dhk;
    MOE_TRY(hip_status(launch_bw_gate_out(go, bf16, s), "backward gate outputs"));
  }
  // 3. score gradients per (token, expert)
  float* dclean = at<float>(ws, L.dclean);
  float* draw = noisy ? at<float>(ws, L.draw) : nullptr;
  float* dbias_part = at<float>(ws, L.dbias_part);
  BwGateArgs ga;
  ga.x = x;
  ga.w_gate = p->w_gate;
  ga.w_noise = noisy ? p->w_noise : nullptr;
  ga.bias = p->bias;
  ga.noise = noisy && n ? noise_src(n, n ? n->eps : nullptr, 0) : NoiseSrc();
  ga.w_pack = p->w_gate_packed;
  ga.pack_nt = gate_pack_tables(c);
  ga.idx = sv->topk_idx;
  ga.thr = smooth ? sv->thr : nullptr;
  ga.dload = smooth ? dload : nullptr;
  ga.dhk = dhk;
  ga.T = T;
  ga.d = d;
  ga.E = E;
  ga.k = k;
  ga.rinfo = at<int32_t>(ws, L.rinfo);
  ga.dclean = dclean;
  ga.draw = draw;
  // bf16 layers: the score gradients leave as the bf16 hi / lo halves the
  // products take (same bytes as fp32, no conversion in the product loaders)
  bf16_t* ch = bf16 ? reinterpret_cast<bf16_t*>(dclean) : nullptr;
  bf16_t* cl = bf16 ? ch + T * E : nullptr;
  bf16_t* rh = bf16 && noisy ? reinterpret_cast<bf16_t*>(draw) : nullptr;
  bf16_t* rl = bf16 && noisy ? rh + T * E : nullptr;
  if (bf16) {
    ga.dclean_hi = ch;
    ga.dclean_lo = cl;
    ga.draw_hi = rh;
    ga.draw_lo = rl;
  }
  ga.dbias_part = dbias_part;
  const bool fused_dxg = L.e16 > 0 && T > 0;
  if (fused_dxg) {
    // the gate's share of dx is formed inside the gate-gradient kernel
    bf16_t* wgt = at<bf16_t>(ws, L.wgt);
    bf16_t* wnt = noisy ? at<bf16_t>(ws, L.wnt) : nullptr;
    MOE_TRY(hip_status(launch_bw_transpose_table(p->w_gate, E, d, L.e16, wgt, s),
                       "backward transpose w_gate"));
    if (noisy)
      MOE_TRY(hip_status(launch_bw_transpose_table(p->w_noise, E, d, L.e16, wnt, s),
                         "backward transpose w_noise"));
    ga.wgt = wgt;
    ga.wnt = wnt;
    ga.e16 = L.e16;
    ga.dxg = dxg;
  }
  MOE_TRY(hip_status(launch_bw_gate(ga, bf16, s), "backward gate"));
  if (g->dbias)
    MOE_TRY(hip_status(launch_bw_sum_rows(dbias_part, L.nblk, E, g->dbias, s), "backward dbias"));
  // 4. gate-table products
  if (T > 0 && !fused_dxg) {
    // bf16 products carry the score gradients as hi + lo halves
    BwGemm q = bf16 ? product(op_rows(ch, E, false), op_cols(p->w_gate, d, false))
                    : product(op_rows(dclean, E, true), op_cols(p->w_gate, d, true));
    q.mode = BW_PLAIN;
    if (bf16) add_pair(q, op_rows(cl, E, false), q.b[0]);
    if (noisy) {
      if (bf16) {
        add_pair(q, op_rows(rh, E, false), op_cols(p->w_noise, d, false));
        add_pair(q, op_rows(rl, E, false), op_cols(p->w_noise, d, false));
      } else {
        add_pair(q, op_rows(draw, E, true), op_cols(p->w_noise, d, true));
      }
    }
    q.M = T;
    q.N = d;
    q.K = E;
    q.kchunk = E;
    q.C = dxg;
    q.c_f32 = 1;
    q.ldc = d;
    const int64_t grid = ((T + 127) / 128) * ((d + 127) / 128);
    MOE_TRY(hip_status(launch_bw_gemm(q, bf16, grid, s), "backward dx gate"));
  }
  if (bf16) {
    MOE_TRY(gate_table_grad_halves(c, L, x, ch, cl, E, g->dw_gate, at<float>(ws, L.part_g),
                                   at<void>(ws, L.zero), s));
    if (noisy)
      MOE_TRY(gate_table_grad_halves(c, L, x, rh, rl, E, g->dw_noise, at<float>(ws, L.part_n),
                                     at<void>(ws, L.zero), s));
  } else {
    MOE_TRY(gate_table_grad(c, L, x, dclean, E, g->dw_gate, at<float>(ws, L.part_g), s));
    if (noisy)
      MOE_TRY(gate_table_grad(c, L, x, draw, E, g->dw_noise, at<float>(ws, L.part_n), s));
  }
  }
  // 6. dx, once the expert side is done
  MOE_TRY(join.wait());
  if (T > 0)
    MOE_TRY(hip_status(launch_bw_assemble_dx(dxg, dxs, sv->inv, T, k, d, bf16, g->dx, s),
                       "backward dx"));
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return layout(cfg).total;
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MOE_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

size_t moe_packed_experts_size(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK || !packable(cfg)) return 0;
  return fused_packed_bytes(cfg->n_experts, cfg->d_model, cfg->d_hidden);
}

moe_status moe_pack_experts(const moe_config* cfg, const moe_params* p, void* packed,
                            void* stream) {
  MOE_TRY(check_config(cfg));
  if (!packable(cfg))
    return fail(MOE_ERR_UNSUPPORTED, "packed expert tables need bf16 ReLU, d_model 512");
  if (!p || !p->w1 || !p->w2 || !packed) return fail(MOE_ERR_INVALID_ARG, "w1 / w2 / packed is NULL");
  if (reinterpret_cast<uintptr_t>(packed) & 15)
    return fail(MOE_ERR_INVALID_ARG, "packed must be 16-byte aligned");
  MOE_TRY(hip_status(launch_pack_experts(p->w1, p->w2, cfg->n_experts, cfg->d_model,
                                         cfg->d_hidden, packed, (hipStream_t)stream),
                     "pack"));
  return ok();
}

size_t moe_packed_gate_size(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK || !gate_packable(cfg)) return 0;
  const int ng = gate_pack_groups(cfg);
  return gate_packed_bytes(ng, cfg->n_experts / ng, cfg->d_model, gate_pack_tables(cfg));
}

moe_status moe_pack_gate(const moe_config* cfg, const moe_params* p, void* packed, void* stream) {
  MOE_TRY(check_config(cfg));
  if (!gate_packable(cfg))
    return fail(MOE_ERR_UNSUPPORTED, "packed gate tables need bf16 and d_model %% 64 == 0");
  if (!p || !p->w_gate || (cfg->noisy && !p->w_noise) || !packed)
    return fail(MOE_ERR_INVALID_ARG, "w_gate / w_noise / packed is NULL");
  if (reinterpret_cast<uintptr_t>(packed) & 15)
    return fail(MOE_ERR_INVALID_ARG, "packed must be 16-byte aligned");
  const int ng = gate_pack_groups(cfg);
  MOE_TRY(hip_status(launch_pack_gate(p->w_gate, p->w_noise, ng, cfg->n_experts / ng,
                                      cfg->d_model, gate_pack_tables(cfg), packed,
                                      (hipStream_t)stream),
                     "pack gate"));
  return ok();
}

moe_status moe_gate(const moe_config* cfg, const void* x, const moe_params* p,
                    const moe_noise* noise, int32_t* topk_idx, float* topk_gate, float* thr,
                    void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_config(cfg));
  MOE_TRY(check_gate_inputs(cfg, x, p, noise));
  if (cfg->tokens > 0 && (!topk_idx || !topk_gate))
    return fail(MOE_ERR_INVALID_ARG, "topk_idx / topk_gate is NULL");
  if (thr && cfg->n_groups > 0) return fail(MOE_ERR_INVALID_ARG, "thr is for the flat gate only");
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  MOE_TRY(do_gate(cfg, layout(cfg), x, p, noise, topk_idx, topk_gate, thr, nullptr, nullptr,
                  nullptr, ws, (hipStream_t)stream));
  return ok();
}

moe_status moe_route(const moe_config* cfg, const int32_t* topk_idx, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* inv, const void* x, void* x_sorted,
                     void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_config(cfg));
  if (!counts || !offsets) return fail(MOE_ERR_INVALID_ARG, "counts / offsets is NULL");
  if (cfg->tokens > 0 && (!topk_idx || !perm || !inv))
    return fail(MOE_ERR_INVALID_ARG, "topk_idx / perm / inv is NULL");
  if ((x == nullptr) != (x_sorted == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "x and x_sorted must be given together");
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  hipStream_t s = (hipStream_t)stream;
  MOE_TRY(do_route(cfg, layout(cfg), topk_idx, counts, offsets, perm, inv, false, false, ws, s));
  if (x)
    MOE_TRY(hip_status(launch_gather_rows(x, perm, cfg->top_k, cfg->tokens * cfg->top_k,
                                          cfg->d_model, (int)elem_size(cfg), x_sorted, s),
                       "gather"));
  return ok();
}

moe_status moe_expert_ffn(const moe_config* cfg, const void* x, const int32_t* perm,
                          const int32_t* offsets, const moe_params* p, void* y_sorted, void* ws,
                          size_t ws_bytes, void* stream) {
  MOE_TRY(check_config(cfg));
  MOE_TRY(check_expert_inputs(cfg, p));
  if (!offsets) return fail(MOE_ERR_INVALID_ARG, "offsets is NULL");
  if (cfg->tokens > 0 && (!x || !y_sorted)) return fail(MOE_ERR_INVALID_ARG, "x / y_sorted is NULL");
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  MOE_TRY(do_ffn(cfg, layout(cfg), x, perm, offsets, p, y_sorted, false, ws,
                 (hipStream_t)stream));
  return ok();
}

moe_status moe_combine(const moe_config* cfg, const void* y_sorted, const int32_t* inv,
                       const float* topk_gate, void* y, void* stream) {
  MOE_TRY(check_config(cfg));
  if (cfg->tokens > 0 && (!y_sorted || !inv || !topk_gate || !y))
    return fail(MOE_ERR_INVALID_ARG, "y_sorted / inv / topk_gate / y is NULL");
  MOE_TRY(hip_status(launch_combine(y_sorted, inv, topk_gate, cfg->tokens, cfg->top_k,
                                    cfg->d_model, cfg->dtype == MOE_BF16, y, (hipStream_t)stream),
                     "combine"));
  return ok();
}

moe_status moe_balance_loss(const moe_config* cfg, const void* x, const moe_params* p,
                            const int32_t* topk_idx, const float* topk_gate, const float* thr,
                            const int32_t* perm, const int32_t* offsets, float w_importance,
                            float w_load, float* importance, float* load, float* out, void* ws,
                            size_t ws_bytes, void* stream) {
  MOE_TRY(check_config(cfg));
  if (!importance || !load || !out || !offsets)
    return fail(MOE_ERR_INVALID_ARG, "importance / load / out / offsets is NULL");
  if (cfg->tokens > 0 && (!perm || !topk_gate))
    return fail(MOE_ERR_INVALID_ARG, "perm / topk_gate is NULL");
  const bool smooth = cfg->n_groups == 0 && cfg->noisy && cfg->tokens > 0;
  if (smooth && (!x || !p || !p->w_gate || !p->w_noise || !topk_idx || !thr))
    return fail(MOE_ERR_INVALID_ARG, "smooth load needs x, w_gate, w_noise, topk_idx and thr");
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  MOE_TRY(do_balance(cfg, layout(cfg), x, p, topk_idx, topk_gate, thr, perm, offsets,
                     w_importance, w_load, importance, load, out, false, ws,
                     (hipStream_t)stream));
  return ok();
}

}  // extern "C"

namespace {

moe_status check_forward_args(const moe_config* cfg, const void* x, const moe_params* p,
                              const moe_noise* noise, const moe_outputs* out) {
  MOE_TRY(check_config(cfg));
  MOE_TRY(check_gate_inputs(cfg, x, p, noise));
  MOE_TRY(check_expert_inputs(cfg, p));
  if (!out || (!out->y && cfg->tokens > 0)) return fail(MOE_ERR_INVALID_ARG, "out / out->y is NULL");
  return MOE_OK;
}

// The layer on a validated call, with its scratch at ws (layout(cfg) bytes).
// side: the smooth-load recompute may run on the device's side stream.
moe_status forward_on(const moe_config* cfg, const void* x, const moe_params* p,
                      const moe_noise* noise, float w_importance, float w_load,
                      moe_outputs* out, void* ws, void* stream, bool side = true) {
  const Layout L = layout(cfg);
  hipStream_t s = (hipStream_t)stream;
  int32_t* idx = out->topk_idx ? out->topk_idx : at<int32_t>(ws, L.idx);
  float* gate = out->topk_gate ? out->topk_gate : at<float>(ws, L.gate);
  int32_t* counts = out->counts ? out->counts : at<int32_t>(ws, L.counts);
  int32_t* offsets = out->offsets ? out->offsets : at<int32_t>(ws, L.offsets);
  int32_t* perm = out->perm ? out->perm : at<int32_t>(ws, L.perm);
  int32_t* inv = out->inv ? out->inv : at<int32_t>(ws, L.inv);
  void* y_sorted = out->y_sorted ? out->y_sorted : at<void>(ws, L.ysorted);
  const bool balance = out->balance != nullptr;
  const bool smooth = balance && cfg->n_groups == 0 && cfg->noisy && cfg->tokens > 0;
  // the flat gate writes the routing masks; the routing step builds the
  // expert tile map
  const bool flat = cfg->n_groups == 0 && cfg->tokens > 0;
  uint32_t* bits = flat ? at<uint32_t>(ws, L.bits) : nullptr;
  const bool tiles = expert_tile_rows(cfg) > 0;
  float* imp = balance ? (out->importance ? out->importance : at<float>(ws, L.imp)) : nullptr;
  float* load = balance ? (out->load ? out->load : at<float>(ws, L.load)) : nullptr;
  // small expert counts: the gate kernel writes per-tile importance (and
  // smooth-load) partials and the routing step reduces them
  const bool fused_stats = balance && flat && gate_fuses_load(cfg->n_experts);
  // thresholds for the smooth-load recompute kernel (or for the caller)
  if (out->thr && cfg->n_groups > 0) return fail(MOE_ERR_INVALID_ARG, "thr is for the flat gate only");
  float* thr = out->thr ? out->thr : (smooth && !fused_stats ? at<float>(ws, L.thr) : nullptr);
  RouteStats st;
  float* part = nullptr;
  if (fused_stats) {
    part = smooth ? at<float>(ws, L.part) : nullptr;
    st.imp_part = at<float>(ws, L.imp_part);
    st.load_part = part;
    st.importance = imp;
    st.load = load;
    st.out = out->balance;
    st.w_imp = w_importance;
    st.w_load = w_load;
  }
  MOE_TRY(do_gate(cfg, L, x, p, noise, idx, gate, thr, part, bits,
                  const_cast<float*>(st.imp_part), ws, s));
  // More than one expert block: the smooth load recomputes the projections
  // (MFMA and VALU work) on the device's side stream, beside the routing and
  // the expert stage (bound by the table stream); the balance reduction
  // waits for both.  The caller's stream waits for the side stream on every
  // return path.
  SideJoin join(s);
  const bool side_load = side && smooth && !fused_stats;
  if (side_load) {
    MOE_TRY(join.fork());
    MOE_TRY(smooth_load_partials(cfg, L, x, p, idx, thr, ws, join.side));
  }
  MOE_TRY(do_route(cfg, L, idx, counts, offsets, perm, inv, flat, tiles, ws, s, st));
  MOE_TRY(do_ffn(cfg, L, x, perm, offsets, p, y_sorted, tiles, ws, s));
  MOE_TRY(hip_status(launch_combine(y_sorted, inv, gate, cfg->tokens, cfg->top_k, cfg->d_model,
                                    cfg->dtype == MOE_BF16, out->y, s),
                     "combine"));
  if (balance && !fused_stats) {
    // the statistics describe the gate's choice: with a capacity they walk
    // the routing without it
    const int32_t* bperm = perm;
    const int32_t* boff = offsets;
    if (cfg->capacity > 0 && cfg->tokens > 0) {
      int32_t* perm_u = at<int32_t>(ws, L.perm_u);
      int32_t* off_u = at<int32_t>(ws, L.offsets_u);
      MOE_TRY(do_route(cfg, L, idx, at<int32_t>(ws, L.counts_u), off_u, perm_u,
                       at<int32_t>(ws, L.inv_u), false, false, ws, s, RouteStats(), false));
      bperm = perm_u;
      boff = off_u;
    }
    if (side_load) {
      MOE_TRY(join.side_follows_main());
      MOE_TRY(do_balance(cfg, L, x, p, idx, gate, thr, bperm, boff, w_importance, w_load, imp,
                         load, out->balance, true, ws, join.side));
      MOE_TRY(join.wait());
    } else {
      MOE_TRY(do_balance(cfg, L, x, p, idx, gate, thr, bperm, boff, w_importance, w_load, imp,
                         load, out->balance, false, ws, s));
    }
  }
  return ok();
}

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[MAX_DEVICES];  // per device, set on its first call

moe_status scratch_ptr(void** ptr) {
  int dev = -1;
  MOE_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= MAX_DEVICES)
    return fail(MOE_ERR_UNSUPPORTED, "device %d is past the %d devices the library tracks", dev,
                MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* a = nullptr;
    MOE_TRY(hip_status(hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)),
                       "hipGetSymbolAddress(scratch)"));
    if (!a || (reinterpret_cast<uintptr_t>(a) & 255))
      return fail(MOE_ERR_HIP, "static scratch of device %d has no usable address", dev);
    g_scratch_ptr[dev] = a;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_config* cfg, const void* x, const moe_params* p,
                       const moe_noise* noise, float w_importance, float w_load, moe_outputs* out,
                       void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_forward_args(cfg, x, p, noise, out));
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  return forward_on(cfg, x, p, noise, w_importance, w_load, out, ws, stream);
}

moe_status moe_forward_static(const moe_config* cfg, const void* x, const moe_params* p,
                              const moe_noise* noise, float w_importance, float w_load,
                              moe_outputs* out, void* stream) {
  MOE_TRY(check_forward_args(cfg, x, p, noise, out));
  const size_t need = layout(cfg).total;
  if (need > MOE_FORWARD_STATIC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "this layer needs %zu bytes of scratch, more than the %zu of the static array "
                "(use moe_forward with a workspace)",
                need, (size_t)MOE_FORWARD_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  MOE_TRY(scratch_ptr(&ws));
  // no side stream: its first use would create it, and the fork and join
  // create events
  return forward_on(cfg, x, p, noise, w_importance, w_load, out, ws, stream, false);
}

// ---- per-batch equal-size mask ---------------------------------------------

}  // extern "C"

namespace {

struct MaskLayout {
  size_t Ht, bits, base, counts, offsets, perm, tokstat, nslot, tok_off, slot_e, slot_g, slot_pos,
      ysorted, hid, tiles, imp, load, bal;
  size_t total;
  int nb;
  int64_t tp, rows;
};

MaskLayout mask_layout(const moe_config* c, int m) {
  MaskLayout L;
  const int64_t T = c->tokens;
  const int E = c->n_experts;
  L.nb = (int)((T + 31) / 32);
  L.tp = 32 * (int64_t)L.nb;
  L.rows = (int64_t)E * m;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  L.Ht = take(4 * (size_t)E * L.tp);
  L.bits = take(4 * (size_t)L.nb * E);
  L.base = take(4 * (size_t)L.nb * E);
  L.counts = take(4 * (size_t)E);
  L.offsets = take(4 * (size_t)(E + 1));
  L.perm = take(4 * (size_t)L.rows);
  L.tokstat = take(8 * (size_t)T);
  L.nslot = take(4 * (size_t)T);
  L.tok_off = take(4 * (size_t)(T + 1));
  L.slot_e = take(4 * (size_t)L.rows);
  L.slot_g = take(4 * (size_t)L.rows);
  L.slot_pos = take(4 * (size_t)L.rows);
  L.ysorted = take(elem_size(c) * (size_t)L.rows * c->d_model);
  const bool fused_ffn = c->dtype == MOE_BF16 &&
                         fused_ffn_supported(c->d_model, c->d_hidden, c->ffn == MOE_FFN_SWIGLU);
  L.hid = take(fused_ffn ? 0 : elem_size(c) * (size_t)L.rows * c->d_hidden);
  L.tiles = take(4 * (size_t)(E + 1));
  L.imp = take(4 * (size_t)E);
  L.load = take(4 * (size_t)E);
  L.bal = take(4 * 4);
  L.total = o;
  return L;
}

moe_status check_mask_request(const moe_config* c, int32_t m) {
  MOE_TRY(check_config(c));
  if (c->n_groups > 0)
    return fail(MOE_ERR_UNSUPPORTED, "the per-batch expert mask is for the flat gate");
  if (c->capacity != 0)
    return fail(MOE_ERR_INVALID_ARG, "capacity must be 0: rows_per_expert sets the rows");
  if (m < 1 || (c->tokens > 0 && m > c->tokens))
    return fail(MOE_ERR_INVALID_ARG, "rows_per_expert must be in [1, tokens]");
  if ((int64_t)c->n_experts * m > (int64_t)INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "n_experts * rows_per_expert exceeds int32 rows");
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_mask_workspace_size(const moe_config* cfg, int32_t rows_per_expert) {
  if (check_mask_request(cfg, rows_per_expert) != MOE_OK) return 0;
  return mask_layout(cfg, rows_per_expert).total;
}

moe_status moe_forward_mask(const moe_config* cfg, const void* x, const moe_params* p,
                            const moe_noise* noise, int32_t rows_per_expert,
                            const float* thresholds, float w_importance, float w_load,
                            moe_mask_outputs* out, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_mask_request(cfg, rows_per_expert));
  MOE_TRY(check_gate_inputs(cfg, x, p, noise));
  MOE_TRY(check_expert_inputs(cfg, p));
  if (!out || (!out->y && cfg->tokens > 0)) return fail(MOE_ERR_INVALID_ARG, "out / out->y is NULL");
  const MaskLayout L = mask_layout(cfg, rows_per_expert);
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", L.total);
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, L.total);
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = cfg->dtype == MOE_BF16;
  const bool noisy = cfg->noisy != 0;
  const int E = cfg->n_experts, m = rows_per_expert;
  int32_t* counts = out->counts ? out->counts : at<int32_t>(ws, L.counts);
  int32_t* offsets = out->offsets ? out->offsets : at<int32_t>(ws, L.offsets);
  int32_t* perm = out->perm ? out->perm : at<int32_t>(ws, L.perm);
  MaskArgs a;
  a.x = x;
  a.w_gate = p->w_gate;
  a.w_noise = noisy ? p->w_noise : nullptr;
  a.bias = p->bias;
  a.noise = noisy ? noise_src(noise, noise ? noise->eps : nullptr, 0) : NoiseSrc();
  a.w_pack = p->w_gate_packed;
  a.pack_nt = gate_pack_tables(cfg);
  a.T = cfg->tokens;
  a.d = cfg->d_model;
  a.E = E;
  a.NB = L.nb;
  a.Tp = L.tp;
  a.m = m;
  a.theta = thresholds;
  a.Ht = at<float>(ws, L.Ht);
  a.bits = at<uint32_t>(ws, L.bits);
  a.base = at<int32_t>(ws, L.base);
  a.offsets = offsets;
  a.tokstat = at<float2>(ws, L.tokstat);
  a.nslot = at<int32_t>(ws, L.nslot);
  a.tok_off = out->tok_offsets ? out->tok_offsets : at<int32_t>(ws, L.tok_off);
  a.slot_e = out->slot_expert ? out->slot_expert : at<int32_t>(ws, L.slot_e);
  a.slot_g = out->slot_gate ? out->slot_gate : at<float>(ws, L.slot_g);
  a.slot_pos = out->slot_row ? out->slot_row : at<int32_t>(ws, L.slot_pos);
  a.importance = out->importance ? out->importance : at<float>(ws, L.imp);
  a.load = out->load ? out->load : at<float>(ws, L.load);
  MOE_TRY(hip_status(launch_mask_scores(a, bf16, noisy, s), "mask scores"));
  if (!thresholds) MOE_TRY(hip_status(launch_mask_select(a, s), "batch mask"));
  RouteArgs r;
  r.idx = nullptr;
  r.T = cfg->tokens;
  r.k = 1;
  r.E = E;
  r.NB = L.nb;
  r.bits = a.bits;
  r.base = at<int32_t>(ws, L.base);
  r.have_bits = 1;
  r.counts = counts;
  r.offsets = offsets;
  r.perm = perm;
  r.inv = nullptr;
  r.tile_rows = 0;
  r.tiles = nullptr;
  r.desc = nullptr;
  r.capacity = m;
  MOE_TRY(hip_status(launch_mask_route(r, L.rows, s), "mask rows"));
  MOE_TRY(hip_status(launch_mask_tokens(a, s), "mask slots"));
  // the experts over the rows: row p is token perm[p]
  moe_config rc = *cfg;
  rc.tokens = L.rows;
  rc.top_k = 1;
  Layout RL{};
  RL.tiles = L.tiles;
  RL.hid = L.hid;
  void* y_sorted = at<void>(ws, L.ysorted);
  MOE_TRY(do_ffn(&rc, RL, x, perm, offsets, p, y_sorted, false, ws, s));
  MOE_TRY(hip_status(launch_combine_csr(y_sorted, a.tok_off, a.slot_pos, a.slot_g, cfg->tokens,
                                        cfg->d_model, bf16, out->y, s),
                     "mask combine"));
  if (out->balance) {
    MOE_TRY(hip_status(launch_mask_balance(a, s), "mask balance"));
    MOE_TRY(hip_status(launch_cv2(a.importance, a.load, E, w_importance, w_load, out->balance, s),
                       "mask cv2"));
  }
  return ok();
}

moe_status moe_draw_noise(const moe_config* cfg, uint64_t seed, float* eps, float* eps_p,
                          void* stream) {
  MOE_TRY(check_config(cfg));
  if (eps_p && cfg->n_groups == 0) return fail(MOE_ERR_INVALID_ARG, "eps_p is for the hierarchy");
  MOE_TRY(hip_status(launch_draw_noise(cfg->tokens, cfg->n_experts, cfg->n_groups, seed, eps, eps_p,
                                       (hipStream_t)stream),
                     "draw noise"));
  return ok();
}

// ---- backward ---------------------------------------------------------------

size_t moe_backward_workspace_size(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return bw_layout(cfg).total;
}

moe_status moe_backward(const moe_config* cfg, const void* x, const moe_params* p,
                        const moe_noise* noise, const moe_saved* sv, const void* dy,
                        float w_importance, float w_load, moe_grads* g, void* ws,
                        size_t ws_bytes, void* stream) {
  MOE_TRY(check_config(cfg));
  if (!p || !sv || !g) return fail(MOE_ERR_INVALID_ARG, "params / saved / grads is NULL");
  const int64_t T = cfg->tokens;
  const bool rows = T > 0;
  const bool noisy = cfg->noisy != 0;
  const bool sw = cfg->ffn == MOE_FFN_SWIGLU;
  const bool hier = cfg->n_groups > 0;
  if (!p->w_gate || (noisy && !p->w_noise))
    return fail(MOE_ERR_INVALID_ARG, "w_gate / w_noise is NULL");
  if (hier) {
    if (!p->w_gate_p || (noisy && !p->w_noise_p))
      return fail(MOE_ERR_INVALID_ARG, "the hierarchy needs w_gate_p (and w_noise_p when noisy)");
    if (p->bias || g->dbias)
      return fail(MOE_ERR_INVALID_ARG, "the hierarchy has no bias (bias / dbias must be NULL)");
    if (g->dw_noise_p && !noisy)
      return fail(MOE_ERR_INVALID_ARG, "dw_noise_p needs a noisy gate");
    if (rows && noisy && !has_noise(noise, noise ? noise->eps_p : nullptr))
      return fail(MOE_ERR_INVALID_ARG, "noisy hierarchy needs eps_p (or noise drawn in the kernels)");
  } else if (g->dw_gate_p || g->dw_noise_p) {
    return fail(MOE_ERR_INVALID_ARG, "dw_gate_p / dw_noise_p are for the hierarchy");
  }
  if (!p->w1 || !p->w2 || (sw && !p->w3))
    return fail(MOE_ERR_INVALID_ARG, "the backward pass needs the unpacked w1 / w2 (/ w3)");
  if (p->w_packed) {
    if (!packable(cfg))
      return fail(MOE_ERR_UNSUPPORTED, "packed expert tables need bf16 ReLU, d_model 512");
    if (reinterpret_cast<uintptr_t>(p->w_packed) & 15)
      return fail(MOE_ERR_INVALID_ARG, "w_packed must be 16-byte aligned");
  }
  if (p->w_gate_packed) {
    if (!gate_packable(cfg))
      return fail(MOE_ERR_UNSUPPORTED, "packed gate tables need bf16 and d_model %% 64 == 0");
    if (reinterpret_cast<uintptr_t>(p->w_gate_packed) & 15)
      return fail(MOE_ERR_INVALID_ARG, "w_gate_packed must be 16-byte aligned");
  }
  if (!g->dx && rows) return fail(MOE_ERR_INVALID_ARG, "grads->dx is NULL");
  if (g->dw_noise && !noisy) return fail(MOE_ERR_INVALID_ARG, "dw_noise needs a noisy gate");
  if (g->dw3 && !sw) return fail(MOE_ERR_INVALID_ARG, "dw3 needs SwiGLU experts");
  if (!sv->offsets) return fail(MOE_ERR_INVALID_ARG, "saved offsets is NULL");
  if (rows) {
    if (!x || !dy) return fail(MOE_ERR_INVALID_ARG, "x / dy is NULL");
    if (noisy && !has_noise(noise, noise ? noise->eps : nullptr))
      return fail(MOE_ERR_INVALID_ARG, "noisy gate needs eps (or noise drawn in the kernels)");
    if (!sv->topk_idx || !sv->topk_gate || !sv->perm || !sv->inv || !sv->y_sorted)
      return fail(MOE_ERR_INVALID_ARG, "saved topk_idx / topk_gate / perm / inv / y_sorted is NULL");
    if (w_importance != 0.f && !sv->importance)
      return fail(MOE_ERR_INVALID_ARG, "w_importance != 0 needs saved importance");
    if (!hier && noisy && w_load != 0.f && (!sv->load || !sv->thr))
      return fail(MOE_ERR_INVALID_ARG, "w_load != 0 with noise needs saved load and thr");
  }
  const BwLayout L = bw_layout(cfg);
  if (L.total > 0) {
    if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", L.total);
    if (reinterpret_cast<uintptr_t>(ws) & 255)
      return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < L.total)
      return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, L.total);
  }
  if (cfg->dtype == MOE_F32 && (cfg->d_model % 4 != 0 || cfg->d_hidden % 4 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "the fp32 backward pass needs d_model and d_hidden multiples of 4");
  if (!hier && bw_gate_lds_bytes(cfg->dtype == MOE_BF16, cfg->d_model, cfg->n_experts) > 150 * 1024)
    return fail(MOE_ERR_UNSUPPORTED, "n_experts / d_model too large for the backward gate tile");
  MOE_TRY(do_backward(cfg, L, x, p, noise, sv, dy, w_importance, w_load, g, ws,
                      (hipStream_t)stream));
  return ok();
}

}  // extern "C"
