// squad_api.hip - the C ABI of libsquad: argument checks, address-map set-up and
// kernel enqueues.  Every check runs on the host before anything is enqueued.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include <rocblas/rocblas.h>

#include "squad.h"
#include "squad_kernels.h"

using namespace squad;

namespace {

struct Geo {
  int64_t T, H, W, tt, th, tw;  // grid and tile
  int64_t nt, nh, nw;           // window grid (cut tilings: rounded up)
  int64_t G, Wn, n;             // windows, tile cells per window, tokens
  bool cut;                     // the grid is not a whole number of tiles
  uint32_t ru = 1;              // row unit of the maps: 1 (narrow) or head_dim (wide)
};

// cut: whether the entry point accepts grids that are not a whole number of tiles
// (read as padded up to one with absent tokens; only the forward family does)
int make_geo(const int32_t grid[3], const int32_t tile[3], Geo& g, bool cut = false) {
  if (!grid || !tile) return SQUAD_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i)
    if (grid[i] <= 0 || tile[i] <= 0) return SQUAD_ERR_INVALID_ARG;
  g.T = grid[0]; g.H = grid[1]; g.W = grid[2];
  g.tt = tile[0]; g.th = tile[1]; g.tw = tile[2];
  g.cut = g.T % g.tt || g.H % g.th || g.W % g.tw;
  if (g.cut && !cut) return SQUAD_ERR_SHAPE;
  if (g.tt > g.T || g.th > g.H || g.tw > g.W) return SQUAD_ERR_SHAPE;
  g.nt = (g.T + g.tt - 1) / g.tt; g.nh = (g.H + g.th - 1) / g.th; g.nw = (g.W + g.tw - 1) / g.tw;
  g.n = g.T * g.H * g.W;
  g.Wn = g.tt * g.th * g.tw;
  g.G = g.nt * g.nh * g.nw;
  if (g.G * g.Wn >= (int64_t(1) << 31)) return SQUAD_ERR_SHAPE;
  return SQUAD_OK;
}

int check_common(int32_t heads, int32_t batch, int32_t head_dim, int32_t dtype) {
  if (heads <= 0 || batch <= 0 || head_dim <= 0) return SQUAD_ERR_INVALID_ARG;
  if (dtype != SQUAD_DTYPE_F32 && dtype != SQUAD_DTYPE_BF16) return SQUAD_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return SQUAD_ERR_UNSUPPORTED;
  return SQUAD_OK;
}

size_t elem_bytes(int32_t dtype) { return dtype == SQUAD_DTYPE_F32 ? 4 : 2; }

bool misaligned(const void* p) { return ((uintptr_t)p & 15) != 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

Mix mix(uint32_t x1, uint32_t x0, int64_t s2, int64_t s1, int64_t s0) {
  Mix m;
  m.x1 = FastDiv(x1);
  m.x0 = FastDiv(x0);
  m.s2 = s2; m.s1 = s1; m.s0 = s0;
  return m;
}

Mix linear(int64_t stride) { return mix(1, 1, stride, 0, 0); }

// ru: the row unit (strides in elements are divided by it; every stride is a
// multiple of head_dim, so wide maps hold whole head rows).  The strides are kept
// modulo 2^32: every row offset formed from them is below 2^32.
Mix32 mix32(uint32_t x1, uint32_t x0, int64_t s2, int64_t s1, int64_t s0, int64_t ru = 1) {
  Mix32 m;
  m.x1 = FastDiv32(x1);
  m.x0 = FastDiv32(x0);
  m.s2 = (int32_t)(uint32_t)(s2 / ru); m.s1 = (int32_t)(uint32_t)(s1 / ru); m.s0 = (int32_t)(uint32_t)(s0 / ru);
  return m;
}

Mix32 linear32(int64_t stride, int64_t ru = 1) { return mix32(1, 1, stride, 0, 0, ru); }

// Token order [B, n, heads, d]: the window part and the offset part of a token index.
// (nh, nw, strides) of the window digits and (th, tw, strides) of the offset digits.
// ts: elements from one token's row to the next (heads * d for [B, n, heads, d];
// larger when q, k and v are slices of one fused projection output)
RowMap token_map(const Geo& g, int64_t heads, int64_t d, bool by_window, int64_t ts = 0) {
  RowMap m;
  if (ts == 0) ts = heads * d;
  m.sB = g.n * ts;
  m.sH = d;
  const int64_t w2 = g.tt * g.H * g.W * ts, w1 = g.th * g.W * ts, w0 = g.tw * ts;
  const int64_t o2 = g.H * g.W * ts, o1 = g.W * ts, o0 = ts;
  if (by_window) {
    m.unit = mix((uint32_t)g.nh, (uint32_t)g.nw, w2, w1, w0);
    m.row = mix32((uint32_t)g.th, (uint32_t)g.tw, o2, o1, o0, g.ru);
  } else {
    m.unit = mix((uint32_t)g.th, (uint32_t)g.tw, o2, o1, o0);
    m.row = mix32((uint32_t)g.nh, (uint32_t)g.nw, w2, w1, w0, g.ru);
  }
  return m;
}

// Group-major [B, heads, Wn, G, d] (by_window: units are windows, rows offsets).
RowMap group_major_map(const Geo& g, int64_t heads, int64_t d, bool by_window) {
  RowMap m;
  m.sB = heads * g.Wn * g.G * d;
  m.sH = g.Wn * g.G * d;
  m.unit = by_window ? linear(d) : linear(g.G * d);
  m.row = by_window ? linear32(g.G * d, g.ru) : linear32(d, g.ru);
  return m;
}

// Window-major [B, heads, G, Wn, d].
RowMap window_major_map(const Geo& g, int64_t heads, int64_t d, bool by_window) {
  RowMap m;
  m.sB = heads * g.G * g.Wn * d;
  m.sH = g.G * g.Wn * d;
  m.unit = by_window ? linear(g.Wn * d) : linear(d);
  m.row = by_window ? linear32(d, g.ru) : linear32(g.Wn * d, g.ru);
  return m;
}

AttnArgs attn_args(const void* q, const void* k, const void* v, void* o, uint32_t L, uint32_t U,
                   uint32_t heads, uint32_t batch, int32_t head_dim, float scale) {
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.L = L; a.U = U; a.heads = heads; a.BH = heads * batch;
  a.fBH = FastDiv(a.BH);
  a.fHeads = FastDiv(heads);
  a.units = a.BH * U;
  const double s = scale > 0.f ? (double)scale : 1.0 / sqrt((double)head_dim);
  a.c = (float)(s * 1.4426950408889634);  // log2(e)
  a.row_unit = 1;
  return a;
}

int run_attn(AttnArgs a, int32_t head_dim, int32_t dtype, hipStream_t stream,
             VType vtype = VType::kBf16ToBf16) {
  if (a.units == 0 || a.L == 0) return SQUAD_OK;
  a.v_like_k = memcmp(&a.mqk.row, &a.mv.row, sizeof(a.mqk.row)) == 0;
  const hipError_t e = dtype == SQUAD_DTYPE_BF16 ? launch_attn_bf16(a, head_dim, vtype, stream)
                                                 : launch_attn_f32(a, head_dim, stream);
  return e == hipSuccess ? SQUAD_OK : SQUAD_ERR_HIP;
}

// The row unit for tensors of `span` elements per batch element (every row offset of
// a call's maps is below it): narrow below 2^31 elements, else wide, up to 2^32 - 1
// head rows.
int pick_row_unit(Geo& g, uint64_t span, int32_t head_dim) {
  if (span < (uint64_t(1) << 31)) {
    g.ru = 1;
    return SQUAD_OK;
  }
  if ((span + head_dim - 1) / head_dim >= (uint64_t)kNoRow) return SQUAD_ERR_SHAPE;
  g.ru = (uint32_t)head_dim;
  return SQUAD_OK;
}

bool too_many_units(uint64_t bh, uint64_t units_per_bh, uint64_t rows) {
  return bh * units_per_bh >= (uint64_t(1) << 32) || rows >= (uint64_t(1) << 32);
}

// Shared checks of the grid/tile entry points: geometry, dtype, sizes, pointers.
// bytes: one token-order tensor; wbytes: the forward's workspace (the local output
// in group-major order, one row per tile cell, absent cells included).
int check_grid_call(const int32_t grid[3], const int32_t tile[3], int32_t heads, int32_t batch,
                    int32_t head_dim, int32_t dtype, Geo& g, size_t& bytes, size_t* wbytes = nullptr,
                    bool cut = false) {
  int st = make_geo(grid, tile, g, cut);
  if (st) return st;
  st = check_common(heads, batch, head_dim, dtype);
  if (st) return st;
  const uint64_t bh = (uint64_t)heads * (uint64_t)batch;
  const uint64_t cells = (uint64_t)g.G * (uint64_t)g.Wn;
  if (too_many_units(bh, (uint64_t)(g.G > g.Wn ? g.G : g.Wn), bh * cells)) return SQUAD_ERR_SHAPE;
  // rows inside one batch element are located by 32-bit offsets: in elements while
  // they stay below 2^31 (narrow maps), else in head rows (wide maps)
  st = pick_row_unit(g, cells * (uint64_t)heads * (uint64_t)head_dim, head_dim);
  if (st) return st;
  bytes = (size_t)bh * (size_t)g.n * (size_t)head_dim * elem_bytes(dtype);
  if (wbytes) *wbytes = (size_t)bh * (size_t)cells * (size_t)head_dim * elem_bytes(dtype);
  return SQUAD_OK;
}

int check_ptrs(const void* const* in, int nin, const void* out, size_t bytes) {
  for (int i = 0; i < nin; ++i)
    if (!in[i]) return SQUAD_ERR_INVALID_ARG;
  if (!out) return SQUAD_ERR_INVALID_ARG;
  for (int i = 0; i < nin; ++i)
    if (misaligned(in[i])) return SQUAD_ERR_ALIGN;
  if (misaligned(out)) return SQUAD_ERR_ALIGN;
  for (int i = 0; i < nin; ++i)
    if (overlap(in[i], bytes, out, bytes)) return SQUAD_ERR_ALIAS;
  return SQUAD_OK;
}

int run_copy(const void* src, void* dst, const RowMap& ms, const RowMap& md, uint32_t L, uint32_t U,
             uint32_t heads, uint32_t batch, int32_t head_dim, int32_t dtype, uint32_t ru, hipStream_t stream) {
  CopyArgs c;
  memset(&c, 0, sizeof(c));
  c.src = src; c.dst = dst; c.ms = ms; c.md = md;
  c.row_unit = ru;
  c.L = L; c.U = U; c.heads = heads; c.BH = heads * batch;
  c.fL = FastDiv(L); c.fU = FastDiv(U); c.fHeads = FastDiv(heads);
  c.rows = c.BH * U * L;
  c.elem_bytes = (uint32_t)elem_bytes(dtype);
  const uint32_t chunks = (uint32_t)(head_dim * c.elem_bytes / 16);
  c.row_chunks_log2 = 0;
  while ((1u << c.row_chunks_log2) < chunks) ++c.row_chunks_log2;
  if (((uint64_t)c.rows << c.row_chunks_log2) >= (uint64_t(1) << 40)) return SQUAD_ERR_SHAPE;
  return launch_row_copy(c, stream) == hipSuccess ? SQUAD_OK : SQUAD_ERR_HIP;
}

}  // namespace

extern "C" {

const char* squad_status_string(int status) {
  switch (status) {
    case SQUAD_OK: return "ok";
    case SQUAD_ERR_INVALID_ARG: return "invalid argument (null pointer, size <= 0 or unknown selector)";
    case SQUAD_ERR_SHAPE: return "shape error (grid not a whole number of tiles, or sizes too large)";
    case SQUAD_ERR_UNSUPPORTED: return "unsupported (head_dim must be 64 or 128; dtype 0 = fp32, 1 = bf16)";
    case SQUAD_ERR_ALIAS: return "an output overlaps an input or the workspace";
    case SQUAD_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
    case SQUAD_ERR_WORKSPACE: return "workspace null or smaller than squad_attn_workspace_size()";
    case SQUAD_ERR_HIP: return "HIP error (no device, or a launch failed)";
    case SQUAD_ERR_SCRATCH:
      return "the local output of one (batch, head) exceeds the no-allocation entry point's "
             "scratch (SQUAD_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t squad_attn_workspace_size(const int32_t grid[3], const int32_t tile[3], int32_t heads,
                                 int32_t batch, int32_t head_dim, int32_t dtype) {
  Geo g;
  size_t bytes = 0, wbytes = 0;
  if (check_grid_call(grid, tile, heads, batch, head_dim, dtype, g, bytes, &wbytes, true)) return 0;
  return wbytes;
}

}  // extern "C"

namespace {

// Checks shared by squad_attn_forward and its two halves: `in` holds the nin input
// pointers, `out` is null for the local half (whose only output is the workspace).
int check_forward(const void* const* in, int nin, const void* out, const int32_t grid[3],
                  const int32_t tile[3], int32_t heads, int32_t batch, int32_t head_dim, int32_t dtype,
                  float scale, const void* workspace, size_t workspace_bytes, Geo& g) {
  size_t bytes = 0, wbytes = 0;
  int st = check_grid_call(grid, tile, heads, batch, head_dim, dtype, g, bytes, &wbytes, true);
  if (st) return st;
  for (int i = 0; i < nin; ++i)
    if (!in[i]) return SQUAD_ERR_INVALID_ARG;
  if (out) {
    st = check_ptrs(in, nin, out, bytes);
    if (st) return st;
  } else {
    for (int i = 0; i < nin; ++i)
      if (misaligned(in[i])) return SQUAD_ERR_ALIGN;
  }
  if (!workspace || workspace_bytes < wbytes) return SQUAD_ERR_WORKSPACE;
  if (misaligned(workspace)) return SQUAD_ERR_ALIGN;
  for (int i = 0; i < nin; ++i)
    if (overlap(in[i], bytes, workspace, wbytes)) return SQUAD_ERR_ALIAS;
  if (out && overlap(out, bytes, workspace, wbytes)) return SQUAD_ERR_ALIAS;
  if (!isfinite(scale)) return SQUAD_ERR_INVALID_ARG;
  return SQUAD_OK;
}

// Cut tilings: a row is present iff its token lies inside the grid.  Token
// coordinate on each axis = window digit * tile size + offset digit; the local
// pass's units are windows (rows offsets), the global pass's the reverse.
// Wide maps are served by the kernels' cut form only: they are marked cut on whole
// tilings too (where every row is present).  Sets the row unit of the maps.
template <typename Args>
void set_cut(Args& a, const Geo& g, bool by_window) {
  a.row_unit = g.ru;
  if (!g.cut && g.ru == 1) return;
  a.cut.on = 1;
  a.cut.lim[0] = (uint32_t)g.T; a.cut.lim[1] = (uint32_t)g.H; a.cut.lim[2] = (uint32_t)g.W;
  const uint32_t tl[3] = {(uint32_t)g.tt, (uint32_t)g.th, (uint32_t)g.tw};
  for (int i = 0; i < 3; ++i) {
    a.cut.su[i] = by_window ? tl[i] : 1;
    a.cut.sr[i] = by_window ? 1 : tl[i];
  }
}

// Local pass of the forward: units = windows, rows = offsets; the output goes to the
// workspace, group-major.  bf16: held as fp16 between the passes (its bf16 rounding
// would take about half of the 1.5e-2 error budget; fp16 costs the same bytes).
int forward_local(const void* q, const void* k, const void* v, const Geo& g, int32_t heads, int32_t batch,
                  int32_t head_dim, int32_t dtype, float scale, void* workspace, hipStream_t s,
                  float* lse = nullptr, int64_t in_ts = 0) {
  AttnArgs a = attn_args(q, k, v, workspace, (uint32_t)g.Wn, (uint32_t)g.G, heads, batch, head_dim, scale);
  a.lse = lse;
  a.mqk = token_map(g, heads, head_dim, true, in_ts);
  a.mv = a.mqk;
  a.mo = group_major_map(g, heads, head_dim, true);
  set_cut(a, g, true);
  return run_attn(a, head_dim, dtype, s, VType::kBf16ToF16);
}

// Global pass of the forward: units = offset groups, rows = windows; the value
// stream is the local output in the workspace; the output goes to token order
// (out_ts: elements from one output token's row to the next, heads * d if 0).
int forward_global(const void* q, const void* k, void* out, const Geo& g, int32_t heads, int32_t batch,
                   int32_t head_dim, int32_t dtype, float scale, const void* workspace, hipStream_t s,
                   float* lse = nullptr, int64_t in_ts = 0, int64_t out_ts = 0) {
  AttnArgs a = attn_args(q, k, workspace, out, (uint32_t)g.G, (uint32_t)g.Wn, heads, batch, head_dim, scale);
  a.lse = lse;
  a.mqk = token_map(g, heads, head_dim, false, in_ts);
  a.mv = group_major_map(g, heads, head_dim, false);
  a.mo = token_map(g, heads, head_dim, false, out_ts);
  set_cut(a, g, false);
  return run_attn(a, head_dim, dtype, s, VType::kF16ToBf16);
}

// ---- training: the forward's saved state and the backward's scratch, in one
// workspace (sections 256-byte aligned)
struct TrainLayout {
  size_t o1, lse_l, lse_g, dsum, dsum_l, do1, dq_sc, dk_sc, total;
};

TrainLayout train_layout(const Geo& g, int32_t heads, int32_t batch, int32_t head_dim, int32_t dtype) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t bh = (size_t)heads * (size_t)batch;
  const size_t cells = (size_t)g.G * (size_t)g.Wn;   // rows of one pass per (batch, head)
  const size_t esz = elem_bytes(dtype);
  TrainLayout t;
  t.o1 = 0;
  t.lse_l = al(t.o1 + bh * cells * head_dim * esz);
  t.lse_g = al(t.lse_l + bh * cells * 4);
  t.dsum = al(t.lse_g + bh * cells * 4);
  t.dsum_l = al(t.dsum + bh * cells * 4);
  t.do1 = al(t.dsum_l + bh * cells * 4);
  size_t end = al(t.do1 + bh * cells * head_dim * esz);
  // bf16 calls hand the global pass's dq and dk parts to the local pass in dq and dk
  // themselves, as scaled fp16 rows: one inverse scale per head row of each (fp32
  // calls sum in dq and dk directly)
  t.dq_sc = t.dk_sc = 0;
  if (dtype == SQUAD_DTYPE_BF16) {
    t.dq_sc = end;
    t.dk_sc = al(t.dq_sc + bh * (size_t)g.n * 4);
    end = al(t.dk_sc + bh * (size_t)g.n * 4);
  }
  t.total = end;
  return t;
}

BwdArgs bwd_args(const Geo& g, bool local, int32_t heads, int32_t batch, int32_t head_dim, float scale) {
  BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.L = (uint32_t)(local ? g.Wn : g.G);
  a.U = (uint32_t)(local ? g.G : g.Wn);
  a.heads = (uint32_t)heads;
  a.BH = (uint32_t)(heads * batch);
  a.fBH = FastDiv(a.BH);
  a.fHeads = FastDiv(a.heads);
  a.units = a.BH * a.U;
  const double sc = scale > 0.f ? (double)scale : 1.0 / sqrt((double)head_dim);
  a.scale = (float)sc;
  a.c = (float)(sc * 1.4426950408889634);
  set_cut(a, g, local);
  return a;
}

// ---- k levels: nested tiles ext[1] | ext[2] | ... | ext[k - 1] | grid
constexpr int KMAX = 8;
struct KGeo {
  int k;
  int64_t ext[KMAX + 1][3];   // ext[0] = one cell, ext[k] = the grid
  int64_t n;
};

int make_kgeo(const int32_t grid[3], const int32_t* tiles, int32_t levels, KGeo& kg) {
  if (!grid || levels < 2 || levels > KMAX || !tiles) return SQUAD_ERR_INVALID_ARG;
  kg.k = levels;
  for (int a = 0; a < 3; ++a) {
    kg.ext[0][a] = 1;
    kg.ext[levels][a] = grid[a];
    for (int j = 1; j < levels; ++j) kg.ext[j][a] = tiles[3 * (j - 1) + a];
  }
  for (int j = 0; j <= levels; ++j)
    for (int a = 0; a < 3; ++a)
      if (kg.ext[j][a] <= 0) return SQUAD_ERR_INVALID_ARG;
  for (int j = 0; j < levels; ++j)
    for (int a = 0; a < 3; ++a)
      if (kg.ext[j + 1][a] % kg.ext[j][a]) return SQUAD_ERR_SHAPE;
  kg.n = (int64_t)grid[0] * grid[1] * grid[2];
  if (kg.n >= (int64_t(1) << 31)) return SQUAD_ERR_SHAPE;
  return SQUAD_OK;
}

// Pass j of k levels: rows = the level-j digits, units = (position inside the
// level-j tile, index of the level-(j+1) tile); token-order tensors.
RowMapK kpass_map(const KGeo& kg, int j, int64_t heads, int64_t d) {
  const int64_t H = kg.ext[kg.k][1], W = kg.ext[kg.k][2];
  const int64_t ts = heads * d, Ws = W * ts, Hs = H * Ws;
  const int64_t* lo = kg.ext[j];
  const int64_t* hi = kg.ext[j + 1];
  RowMapK m;
  m.sB = kg.n * ts;
  m.sH = d;
  m.row = mix32((uint32_t)(hi[1] / lo[1]), (uint32_t)(hi[2] / lo[2]), lo[0] * Hs, lo[1] * Ws, lo[2] * ts);
  m.unit = mix((uint32_t)lo[1], (uint32_t)lo[2], Hs, Ws, ts);
  m.outer = mix((uint32_t)(H / hi[1]), (uint32_t)(W / hi[2]), hi[0] * Hs, hi[1] * Ws, hi[2] * ts);
  m.split = FastDiv((uint32_t)(lo[0] * lo[1] * lo[2]));
  return m;
}

int64_t kpass_rows(const KGeo& kg, int j) {
  return (kg.ext[j + 1][0] / kg.ext[j][0]) * (kg.ext[j + 1][1] / kg.ext[j][1]) *
         (kg.ext[j + 1][2] / kg.ext[j][2]);
}

int run_bwd(const BwdArgs& a, int32_t head_dim, int32_t dtype, BwdTypes t, hipStream_t s) {
  if (a.units == 0 || a.L == 0) return SQUAD_OK;
  if (dtype == SQUAD_DTYPE_BF16 && bwd_bf16_fused(a.L, a.cut.on))
    return launch_bwd_bf16_small(a, head_dim, t, s) == hipSuccess ? SQUAD_OK : SQUAD_ERR_HIP;
  for (int kind = 0; kind < 2; ++kind) {
    const hipError_t e = dtype == SQUAD_DTYPE_BF16 ? launch_bwd_bf16(a, head_dim, t, kind == 1, s)
                                                   : launch_bwd_f32(a, head_dim, kind == 1, s);
    if (e != hipSuccess) return SQUAD_ERR_HIP;
  }
  return SQUAD_OK;
}

}  // namespace

extern "C" {

int squad_attn_forward(const void* q, const void* k, const void* v, const int32_t grid[3],
                       const int32_t tile[3], int32_t heads, void* out, int32_t batch,
                       int32_t head_dim, int32_t dtype, float scale, void* workspace,
                       size_t workspace_bytes, squad_stream_t stream) {
  Geo g;
  if (!out) return SQUAD_ERR_INVALID_ARG;
  const void* in[3] = {q, k, v};
  int st = check_forward(in, 3, out, grid, tile, heads, batch, head_dim, dtype, scale, workspace,
                         workspace_bytes, g);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  st = forward_local(q, k, v, g, heads, batch, head_dim, dtype, scale, workspace, s);
  if (st) return st;
  return forward_global(q, k, out, g, heads, batch, head_dim, dtype, scale, workspace, s);
}

int squad_attn_forward_local(const void* q, const void* k, const void* v, const int32_t grid[3],
                             const int32_t tile[3], int32_t heads, int32_t batch, int32_t head_dim,
                             int32_t dtype, float scale, void* workspace, size_t workspace_bytes,
                             squad_stream_t stream) {
  Geo g;
  const void* in[3] = {q, k, v};
  int st = check_forward(in, 3, nullptr, grid, tile, heads, batch, head_dim, dtype, scale, workspace,
                         workspace_bytes, g);
  if (st) return st;
  return forward_local(q, k, v, g, heads, batch, head_dim, dtype, scale, workspace, (hipStream_t)stream);
}

int squad_attn_forward_global(const void* q, const void* k, const int32_t grid[3], const int32_t tile[3],
                              int32_t heads, void* out, int32_t batch, int32_t head_dim, int32_t dtype,
                              float scale, const void* workspace, size_t workspace_bytes,
                              squad_stream_t stream) {
  Geo g;
  if (!out) return SQUAD_ERR_INVALID_ARG;
  const void* in[2] = {q, k};
  int st = check_forward(in, 2, out, grid, tile, heads, batch, head_dim, dtype, scale, workspace,
                         workspace_bytes, g);
  if (st) return st;
  return forward_global(q, k, out, g, heads, batch, head_dim, dtype, scale, workspace, (hipStream_t)stream);
}

int squad_local_pass(const void* q, const void* k, const void* v, const int32_t grid[3],
                     const int32_t tile[3], int32_t heads, void* o1, int32_t batch,
                     int32_t head_dim, int32_t dtype, float scale, squad_stream_t stream) {
  Geo g;
  size_t bytes = 0;
  int st = check_grid_call(grid, tile, heads, batch, head_dim, dtype, g, bytes, nullptr, true);
  if (st) return st;
  const void* in[3] = {q, k, v};
  st = check_ptrs(in, 3, o1, bytes);
  if (st) return st;
  if (!isfinite(scale)) return SQUAD_ERR_INVALID_ARG;
  AttnArgs a = attn_args(q, k, v, o1, (uint32_t)g.Wn, (uint32_t)g.G, heads, batch, head_dim, scale);
  a.mqk = token_map(g, heads, head_dim, true);
  a.mv = a.mqk;
  a.mo = a.mqk;
  set_cut(a, g, true);
  return run_attn(a, head_dim, dtype, (hipStream_t)stream);
}

int squad_global_pass(const void* q, const void* k, const void* vstream, const int32_t grid[3],
                      const int32_t tile[3], int32_t heads, void* out, int32_t batch,
                      int32_t head_dim, int32_t dtype, float scale, squad_stream_t stream) {
  Geo g;
  size_t bytes = 0;
  int st = check_grid_call(grid, tile, heads, batch, head_dim, dtype, g, bytes, nullptr, true);
  if (st) return st;
  const void* in[3] = {q, k, vstream};
  st = check_ptrs(in, 3, out, bytes);
  if (st) return st;
  if (!isfinite(scale)) return SQUAD_ERR_INVALID_ARG;
  AttnArgs a = attn_args(q, k, vstream, out, (uint32_t)g.G, (uint32_t)g.Wn, heads, batch, head_dim, scale);
  a.mqk = token_map(g, heads, head_dim, false);
  a.mv = a.mqk;
  a.mo = a.mqk;
  set_cut(a, g, false);
  return run_attn(a, head_dim, dtype, (hipStream_t)stream);
}

int squad_tile_gather(const void* src, void* dst, const int32_t grid[3], const int32_t tile[3],
                      int32_t heads, int32_t batch, int32_t head_dim, int32_t dtype,
                      squad_stream_t stream) {
  Geo g;
  size_t bytes = 0;
  int st = check_grid_call(grid, tile, heads, batch, head_dim, dtype, g, bytes);
  if (st) return st;
  const void* in[1] = {src};
  st = check_ptrs(in, 1, dst, bytes);
  if (st) return st;
  return run_copy(src, dst, token_map(g, heads, head_dim, true), window_major_map(g, heads, head_dim, true),
                  (uint32_t)g.Wn, (uint32_t)g.G, heads, batch, head_dim, dtype, g.ru, (hipStream_t)stream);
}

int squad_tile_scatter(const void* src, void* dst, const int32_t grid[3], const int32_t tile[3],
                       int32_t heads, int32_t batch, int32_t head_dim, int32_t dtype,
                       squad_stream_t stream) {
  Geo g;
  size_t bytes = 0;
  int st = check_grid_call(grid, tile, heads, batch, head_dim, dtype, g, bytes);
  if (st) return st;
  const void* in[1] = {src};
  st = check_ptrs(in, 1, dst, bytes);
  if (st) return st;
  return run_copy(src, dst, window_major_map(g, heads, head_dim, true), token_map(g, heads, head_dim, true),
                  (uint32_t)g.Wn, (uint32_t)g.G, heads, batch, head_dim, dtype, g.ru, (hipStream_t)stream);
}

int squad_window_to_group(const void* src, void* dst, const int32_t grid[3], const int32_t tile[3],
                          int32_t heads, int32_t batch, int32_t head_dim, int32_t dtype,
                          squad_stream_t stream) {
  Geo g;
  size_t bytes = 0;
  int st = check_grid_call(grid, tile, heads, batch, head_dim, dtype, g, bytes);
  if (st) return st;
  const void* in[1] = {src};
  st = check_ptrs(in, 1, dst, bytes);
  if (st) return st;
  // enumerate rows in the group-major (destination) order: units = offsets, rows = windows
  return run_copy(src, dst, window_major_map(g, heads, head_dim, false), group_major_map(g, heads, head_dim, false),
                  (uint32_t)g.G, (uint32_t)g.Wn, heads, batch, head_dim, dtype, g.ru, (hipStream_t)stream);
}

int squad_window_attn(const void* q, const void* k, const void* v, void* out, int32_t units,
                      int32_t len, int32_t head_dim, int32_t dtype, float scale,
                      squad_stream_t stream) {
  if (units <= 0 || len <= 0) return SQUAD_ERR_INVALID_ARG;
  int st = check_common(1, 1, head_dim, dtype);
  if (st) return st;
  if ((uint64_t)len * (uint64_t)head_dim >= (uint64_t(1) << 31)) return SQUAD_ERR_SHAPE;
  const size_t bytes = (size_t)units * (size_t)len * (size_t)head_dim * elem_bytes(dtype);
  const void* in[3] = {q, k, v};
  st = check_ptrs(in, 3, out, bytes);
  if (st) return st;
  if (!isfinite(scale)) return SQUAD_ERR_INVALID_ARG;
  AttnArgs a = attn_args(q, k, v, out, (uint32_t)len, (uint32_t)units, 1, 1, head_dim, scale);
  RowMap m;
  m.sB = 0; m.sH = 0;
  m.unit = linear((int64_t)len * head_dim);
  m.row = linear32(head_dim);
  a.mqk = m; a.mv = m; a.mo = m;
  return run_attn(a, head_dim, dtype, (hipStream_t)stream);
}

int squad_dense_attn_forward(const void* q, const void* k, const void* v, void* out, int32_t batch,
                             int32_t n, int32_t heads, int32_t head_dim, int32_t dtype, float scale,
                             squad_stream_t stream) {
  if (n <= 0) return SQUAD_ERR_INVALID_ARG;
  int st = check_common(heads, batch, head_dim, dtype);
  if (st) return st;
  if ((uint64_t)batch * (uint64_t)heads >= (uint64_t(1) << 32)) return SQUAD_ERR_SHAPE;
  if ((uint64_t)n * (uint64_t)heads * (uint64_t)head_dim >= (uint64_t(1) << 31)) return SQUAD_ERR_SHAPE;
  const size_t bytes = (size_t)batch * (size_t)n * (size_t)heads * (size_t)head_dim * elem_bytes(dtype);
  const void* in[3] = {q, k, v};
  st = check_ptrs(in, 3, out, bytes);
  if (st) return st;
  if (!isfinite(scale)) return SQUAD_ERR_INVALID_ARG;
  AttnArgs a = attn_args(q, k, v, out, (uint32_t)n, 1, heads, batch, head_dim, scale);
  RowMap m;
  m.sB = (int64_t)n * heads * head_dim;
  m.sH = head_dim;
  m.unit = linear(0);
  m.row = linear32((int64_t)heads * head_dim);
  a.mqk = m; a.mv = m; a.mo = m;
  return run_attn(a, head_dim, dtype, (hipStream_t)stream);
}

int squad_plan_tile(const int32_t grid[3], int32_t tile_out[3]) {
  if (!grid || !tile_out) return SQUAD_ERR_INVALID_ARG;
  for (int i = 0; i < 3; ++i)
    if (grid[i] <= 0) return SQUAD_ERR_INVALID_ARG;
  const uint64_t n = (uint64_t)grid[0] * (uint64_t)grid[1] * (uint64_t)grid[2];
  if (n >= (uint64_t(1) << 31)) return SQUAD_ERR_SHAPE;
  // per axis, the smallest tile for each number of windows k: ceil(X / k)
  std::vector<int64_t> cand[3];
  for (int i = 0; i < 3; ++i) {
    const int64_t X = grid[i];
    for (int64_t k = 1; k <= X; ++k) {
      const int64_t t = (X + k - 1) / k;
      if (cand[i].empty() || cand[i].back() != t) cand[i].push_back(t);
      // beyond sqrt(X) consecutive k give the same t; jump to the next change
      if (t > 1) k = std::max(k, (X + t - 2) / (t - 1) - 1);
    }
    std::sort(cand[i].begin(), cand[i].end());
    cand[i].erase(std::unique(cand[i].begin(), cand[i].end()), cand[i].end());
  }
  // ties: fewer absent tokens, then the most compact window (along every axis the
  // tile extent closest to the number of windows, in log ratio), then the first in
  // ascending (tt, th, tw) order
  uint64_t best_cost = ~uint64_t(0), best_pad = ~uint64_t(0);
  double best_skew = 0.0;
  int64_t best[3] = {grid[0], grid[1], grid[2]};
  for (int64_t tt : cand[0])
    for (int64_t th : cand[1])
      for (int64_t tw : cand[2]) {
        const int64_t t[3] = {tt, th, tw};
        uint64_t wn = 1, gp = 1;
        double skew = 0.0;
        for (int i = 0; i < 3; ++i) {
          const int64_t k = (grid[i] + t[i] - 1) / t[i];
          wn *= (uint64_t)t[i];
          gp *= (uint64_t)k;
          const double l = std::log((double)t[i] / (double)k);
          skew += l * l;
        }
        const uint64_t cost = gp * wn * (wn + gp);
        const uint64_t pad = gp * wn - n;
        const bool better = cost != best_cost ? cost < best_cost
                          : pad != best_pad   ? pad < best_pad
                                              : skew < best_skew - 1e-12;
        if (better) {
          best_cost = cost;
          best_pad = pad;
          best_skew = skew;
          best[0] = tt; best[1] = th; best[2] = tw;
        }
      }
  for (int i = 0; i < 3; ++i) tile_out[i] = (int32_t)best[i];
  return SQUAD_OK;
}

int squad_debug_row_offsets(int32_t which, const int32_t grid[3], const int32_t tile[3], int32_t heads,
                            int32_t batch, int32_t head_dim, int64_t* offsets) {
  Geo g;
  size_t bytes = 0;
  int st = check_grid_call(grid, tile, heads, batch, head_dim, SQUAD_DTYPE_F32, g, bytes, nullptr, true);
  if (st) return st;
  if (!offsets) return SQUAD_ERR_INVALID_ARG;
  RowMap m;
  uint32_t U, L;
  switch (which) {
    case 0: m = token_map(g, heads, head_dim, true); U = (uint32_t)g.G; L = (uint32_t)g.Wn; break;
    case 1: m = token_map(g, heads, head_dim, false); U = (uint32_t)g.Wn; L = (uint32_t)g.G; break;
    case 2: m = group_major_map(g, heads, head_dim, true); U = (uint32_t)g.G; L = (uint32_t)g.Wn; break;
    case 3: m = group_major_map(g, heads, head_dim, false); U = (uint32_t)g.Wn; L = (uint32_t)g.G; break;
    default: return SQUAD_ERR_INVALID_ARG;
  }
  // the token maps of a cut tiling: absent rows read -1, through the kernels' own test
  AttnArgs a{};
  a.mqk = m;
  if (which < 2) set_cut(a, g, which == 0);
  size_t i = 0;
  for (uint32_t b = 0; b < (uint32_t)batch; ++b)
    for (uint32_t h = 0; h < (uint32_t)heads; ++h)
      for (uint32_t s = 0; s < U; ++s) {
        const int64_t base = m.base(b, h, s);
        const UnitDigits ud = cut_unit_digits(a, s);
        for (uint32_t r = 0; r < L; ++r)
          offsets[i++] = (!a.cut.on || cut_present(a, ud, r)) ? base + (int64_t)row_elems_rt(m.row_off(r), g.ru)
                                                                : -1;
      }
  return SQUAD_OK;
}

// ---- training forward and backward

size_t squad_attn_train_workspace_size(const int32_t grid[3], const int32_t tile[3], int32_t heads,
                                       int32_t batch, int32_t head_dim, int32_t dtype) {
  Geo g;
  size_t bytes = 0;
  if (check_grid_call(grid, tile, heads, batch, head_dim, dtype, g, bytes, nullptr, true)) return 0;
  return train_layout(g, heads, batch, head_dim, dtype).total;
}

int squad_attn_forward_train(const void* q, const void* k, const void* v, const int32_t grid[3],
                             const int32_t tile[3], int32_t heads, void* out, int32_t batch,
                             int32_t head_dim, int32_t dtype, float scale, void* workspace,
                             size_t workspace_bytes, squad_stream_t stream) {
  Geo g;
  if (!out) return SQUAD_ERR_INVALID_ARG;
  const void* in[3] = {q, k, v};
  int st = check_forward(in, 3, out, grid, tile, heads, batch, head_dim, dtype, scale, workspace,
                         workspace_bytes, g);
  if (st) return st;
  const TrainLayout t = train_layout(g, heads, batch, head_dim, dtype);
  if (workspace_bytes < t.total) return SQUAD_ERR_WORKSPACE;
  size_t bytes = (size_t)heads * batch * g.n * head_dim * elem_bytes(dtype);
  for (int i = 0; i < 3; ++i)
    if (overlap(in[i], bytes, workspace, t.total)) return SQUAD_ERR_ALIAS;
  if (overlap(out, bytes, workspace, t.total)) return SQUAD_ERR_ALIAS;
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  st = forward_local(q, k, v, g, heads, batch, head_dim, dtype, scale, ws + t.o1, s, (float*)(ws + t.lse_l));
  if (st) return st;
  return forward_global(q, k, out, g, heads, batch, head_dim, dtype, scale, ws + t.o1, s,
                        (float*)(ws + t.lse_g));
}

int squad_attn_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const int32_t grid[3], const int32_t tile[3], int32_t heads, void* dq, void* dk,
                        void* dv, int32_t batch, int32_t head_dim, int32_t dtype, float scale,
                        void* workspace, size_t workspace_bytes, squad_stream_t stream) {
  Geo g;
  size_t bytes = 0;
  int st = check_grid_call(grid, tile, heads, batch, head_dim, dtype, g, bytes, nullptr, true);
  if (st) return st;
  const void* in[5] = {q, k, v, out, dout};
  void* outs[3] = {dq, dk, dv};
  for (const void* p : in)
    if (!p) return SQUAD_ERR_INVALID_ARG;
  for (const void* p : outs)
    if (!p) return SQUAD_ERR_INVALID_ARG;
  if (!workspace) return SQUAD_ERR_WORKSPACE;
  for (const void* p : in)
    if (misaligned(p)) return SQUAD_ERR_ALIGN;
  for (const void* p : outs)
    if (misaligned(p)) return SQUAD_ERR_ALIGN;
  if (misaligned(workspace)) return SQUAD_ERR_ALIGN;
  const TrainLayout t = train_layout(g, heads, batch, head_dim, dtype);
  if (workspace_bytes < t.total) return SQUAD_ERR_WORKSPACE;
  for (int i = 0; i < 3; ++i) {
    for (const void* p : in)
      if (overlap(outs[i], bytes, p, bytes)) return SQUAD_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], bytes, outs[j], bytes)) return SQUAD_ERR_ALIAS;
    if (overlap(outs[i], bytes, workspace, t.total)) return SQUAD_ERR_ALIAS;
  }
  for (const void* p : in)
    if (overlap(p, bytes, workspace, t.total)) return SQUAD_ERR_ALIAS;
  if (!isfinite(scale)) return SQUAD_ERR_INVALID_ARG;

  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = dtype == SQUAD_DTYPE_BF16;
  // fp32: dq and dk accumulate in place; bf16: the global pass's parts travel in dq
  // and dk as scaled fp16 rows (2^-12 of the row's largest magnitude at most)
  float* dq_acc = bf16 ? nullptr : (float*)dq;
  float* dk_acc = bf16 ? nullptr : (float*)dk;
  float* dq_sc = bf16 ? (float*)(ws + t.dq_sc) : nullptr;
  float* dk_sc = bf16 ? (float*)(ws + t.dk_sc) : nullptr;

  // global pass: units = offset groups, values = the local output; its value
  // gradient (the local output's gradient) goes to the workspace, group-major
  BwdArgs ag = bwd_args(g, false, heads, batch, head_dim, scale);
  ag.q = q; ag.k = k; ag.v = ws + t.o1; ag.o = out; ag.dout = dout;
  ag.mqk = token_map(g, heads, head_dim, false);
  ag.mv = group_major_map(g, heads, head_dim, false);
  ag.mo = ag.mqk; ag.mdo = ag.mqk;
  ag.lse = (const float*)(ws + t.lse_g);
  ag.dsum = (float*)(ws + t.dsum);
  ag.dq = dq; ag.dk = dk; ag.dq_acc = dq_acc; ag.dk_acc = dk_acc; ag.dq_sc = dq_sc; ag.dk_sc = dk_sc;
  ag.mdq = ag.mqk; ag.mdk = ag.mqk;
  ag.dv = ws + t.do1; ag.mdv = ag.mv;
  ag.final_pass = bf16 ? kPartWrite : kAccWrite;
  // the global pass's key side (bf16, when it runs as the two kinds) also leaves D
  // of the local pass, <do1, o1>, for the rows of every window; the local pass's
  // query side then reads it instead of the local output
  const bool hand_off = bf16 && !bwd_bf16_fused(ag.L, ag.cut.on) && !bwd_bf16_fused(g.Wn, g.cut || g.ru > 1);
  if (hand_off) ag.dsum_next = (float*)(ws + t.dsum_l);
  st = run_bwd(ag, head_dim, dtype, BwdTypes{true, false}, s);
  if (st) return st;

  // local pass: units = windows, upstream gradient = the local output's gradient;
  // adds the global pass's dq and dk and writes the three gradients
  BwdArgs al = bwd_args(g, true, heads, batch, head_dim, scale);
  al.q = q; al.k = k; al.v = v; al.o = ws + t.o1; al.dout = ws + t.do1;
  al.mqk = token_map(g, heads, head_dim, true);
  al.mv = al.mqk;
  al.mo = group_major_map(g, heads, head_dim, true);
  al.mdo = al.mo;
  al.lse = (const float*)(ws + t.lse_l);
  al.dsum = (float*)(ws + (hand_off ? t.dsum_l : t.dsum));
  al.dsum_ready = hand_off ? 1 : 0;
  al.dq = dq; al.dk = dk; al.dq_acc = dq_acc; al.dk_acc = dk_acc; al.dq_sc = dq_sc; al.dk_sc = dk_sc;
  al.mdq = al.mqk; al.mdk = al.mqk;
  al.dv = dv; al.mdv = al.mqk;
  al.final_pass = bf16 ? kPartFinal : kAccFinal;
  return run_bwd(al, head_dim, dtype, BwdTypes{false, true}, s);
}

// ---- more than two passes

size_t squad_kpass_workspace_size(const int32_t grid[3], const int32_t* tiles, int32_t levels, int32_t heads,
                                  int32_t batch, int32_t head_dim, int32_t dtype) {
  KGeo kg;
  if (make_kgeo(grid, tiles, levels, kg) || check_common(heads, batch, head_dim, dtype)) return 0;
  const size_t one = (size_t)heads * batch * kg.n * head_dim * (dtype == SQUAD_DTYPE_BF16 ? 2 : 4);
  return levels > 2 ? 2 * one : one;
}

}  // extern "C"

namespace {

// Shape checks of the k-level entry points.
int kpass_check(const int32_t grid[3], const int32_t* tiles, int32_t levels, int32_t heads, int32_t batch,
                int32_t head_dim, int32_t dtype, KGeo& kg) {
  int st = make_kgeo(grid, tiles, levels, kg);
  if (st) return st;
  st = check_common(heads, batch, head_dim, dtype);
  if (st) return st;
  const uint64_t bh = (uint64_t)heads * (uint64_t)batch;
  if ((uint64_t)kg.n * (uint64_t)heads * (uint64_t)head_dim >= (uint64_t(1) << 31)) return SQUAD_ERR_SHAPE;
  for (int j = 0; j < levels; ++j)
    if (too_many_units(bh, (uint64_t)(kg.n / kpass_rows(kg, j)), bh * (uint64_t)kg.n)) return SQUAD_ERR_SHAPE;
  return SQUAD_OK;
}

// Level j's token maps when it is the first or the last level: the two-pass
// operator's local pass (tile = the level-1 tile) or global pass (tile = the
// level-(k-1) tile).
int kpass_end_map(const KGeo& kg, const int32_t grid[3], int j, int32_t heads, int32_t head_dim, RowMap& m) {
  Geo g;
  const int ti = j == 0 ? 1 : kg.k - 1;
  const int32_t tile[3] = {(int32_t)kg.ext[ti][0], (int32_t)kg.ext[ti][1], (int32_t)kg.ext[ti][2]};
  const int st = make_geo(grid, tile, g);
  if (st) return st;
  m = token_map(g, heads, head_dim, j == 0);
  return SQUAD_OK;
}

// The k levels of the forward: level j reads its values from v (j = 0) or
// level_out[j - 1] and writes level_out[j] (out for the last level); lse_base
// (optional) receives each level's row statistics, batch*heads*n floats per level.
int kpass_levels_forward(const void* q, const void* k, const void* v, const KGeo& kg, const int32_t grid[3],
                         int32_t heads, void* out, int32_t batch, int32_t head_dim, int32_t dtype, float scale,
                         void* const* level_out, float* lse_base, hipStream_t s) {
  const int levels = kg.k;
  const size_t rows = (size_t)heads * batch * kg.n;
  const bool bf16 = dtype == SQUAD_DTYPE_BF16;
  for (int j = 0; j < levels; ++j) {
    const uint32_t L = (uint32_t)kpass_rows(kg, j);
    const uint32_t U = (uint32_t)(kg.n / L);
    const void* vin = j == 0 ? v : level_out[j - 1];
    void* o = j == levels - 1 ? out : level_out[j];
    float* lse = lse_base ? lse_base + (size_t)j * rows : nullptr;
    int st;
    if (j == 0 || j == levels - 1) {
      AttnArgs a = attn_args(q, k, vin, o, L, U, heads, batch, head_dim, scale);
      st = kpass_end_map(kg, grid, j, heads, head_dim, a.mqk);
      if (st) return st;
      a.mv = a.mqk;
      a.mo = a.mqk;
      a.lse = lse;
      const VType vt = j == 0 ? VType::kBf16ToF16 : VType::kF16ToBf16;
      st = run_attn(a, head_dim, dtype, s, vt);
    } else {
      const AttnArgs base = attn_args(q, k, vin, o, L, U, heads, batch, head_dim, scale);
      AttnArgsK a;
      memset(&a, 0, sizeof(a));
      a.q = base.q; a.k = base.k; a.v = base.v; a.o = base.o;
      a.L = base.L; a.U = base.U; a.heads = base.heads; a.BH = base.BH;
      a.fBH = base.fBH; a.fHeads = base.fHeads; a.units = base.units; a.c = base.c;
      a.mqk = kpass_map(kg, j, heads, head_dim);
      a.mv = a.mqk;
      a.mo = a.mqk;
      a.v_like_k = 1;
      a.lse = lse;
      if (a.units == 0) continue;
      const hipError_t e = bf16 ? launch_attn_bf16_k(a, head_dim, s) : launch_attn_f32_k(a, head_dim, s);
      st = e == hipSuccess ? SQUAD_OK : SQUAD_ERR_HIP;
    }
    if (st) return st;
  }
  return SQUAD_OK;
}

// Training workspace of k levels (sections 256-byte aligned): the intermediate
// outputs o_1 .. o_(k-1) (fp16 for bf16 calls), each level's row statistics, D,
// two buffers for the intermediate outputs' gradients (the call's dtype), and for
// bf16 calls the fp32 sums of dq and dk.
struct KTrainLayout {
  size_t inter, lse, dsum, dgrad[2], dq_acc, dk_acc, dq_sc, dk_sc, one_i, one_g, total;
};

KTrainLayout kpass_train_layout(const KGeo& kg, int32_t heads, int32_t batch, int32_t head_dim, int32_t dtype) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows = (size_t)heads * batch * kg.n;
  const bool bf16 = dtype == SQUAD_DTYPE_BF16;
  KTrainLayout t;
  t.one_i = al(rows * head_dim * (bf16 ? 2 : 4));
  t.one_g = al(rows * head_dim * elem_bytes(dtype));
  t.inter = 0;
  t.lse = t.inter + (size_t)(kg.k - 1) * t.one_i;
  t.dsum = al(t.lse + (size_t)kg.k * rows * 4);
  t.dgrad[0] = al(t.dsum + rows * 4);
  t.dgrad[1] = t.dgrad[0] + t.one_g;
  size_t end = t.dgrad[1] + t.one_g;
  // bf16: the levels' dq and dk parts travel in dq and dk as scaled fp16 rows, as
  // in squad_attn_backward (one inverse scale per head row); the middle levels add
  // to them
  t.dq_acc = t.dk_acc = t.dq_sc = t.dk_sc = 0;
  if (bf16) {
    t.dq_sc = end;
    t.dk_sc = al(t.dq_sc + rows * 4);
    end = al(t.dk_sc + rows * 4);
  }
  t.total = end;
  return t;
}

template <typename Args>
void kpass_bwd_common(Args& a, const KGeo& kg, int j, int32_t heads, int32_t batch, int32_t head_dim, float scale) {
  a.L = (uint32_t)kpass_rows(kg, j);
  a.U = (uint32_t)(kg.n / a.L);
  a.heads = (uint32_t)heads;
  a.BH = (uint32_t)(heads * batch);
  a.fBH = FastDiv(a.BH);
  a.fHeads = FastDiv(a.heads);
  a.units = a.BH * a.U;
  const double sc = scale > 0.f ? (double)scale : 1.0 / sqrt((double)head_dim);
  a.scale = (float)sc;
  a.c = (float)(sc * 1.4426950408889634);
}

}  // namespace

extern "C" {

int squad_kpass_forward(const void* q, const void* k, const void* v, const int32_t grid[3],
                        const int32_t* tiles, int32_t levels, int32_t heads, void* out, int32_t batch,
                        int32_t head_dim, int32_t dtype, float scale, void* workspace,
                        size_t workspace_bytes, squad_stream_t stream) {
  KGeo kg;
  int st = kpass_check(grid, tiles, levels, heads, batch, head_dim, dtype, kg);
  if (st) return st;
  const uint64_t bh = (uint64_t)heads * (uint64_t)batch;
  const size_t bytes = (size_t)bh * kg.n * head_dim * elem_bytes(dtype);
  const void* in[3] = {q, k, v};
  st = check_ptrs(in, 3, out, bytes);
  if (st) return st;
  const size_t one = (size_t)bh * kg.n * head_dim * (dtype == SQUAD_DTYPE_BF16 ? 2 : 4);
  const size_t need = levels > 2 ? 2 * one : one;
  if (!workspace || workspace_bytes < need) return SQUAD_ERR_WORKSPACE;
  if (misaligned(workspace)) return SQUAD_ERR_ALIGN;
  for (int i = 0; i < 3; ++i)
    if (overlap(in[i], bytes, workspace, need)) return SQUAD_ERR_ALIAS;
  if (overlap(out, bytes, workspace, need)) return SQUAD_ERR_ALIAS;
  if (!isfinite(scale)) return SQUAD_ERR_INVALID_ARG;
  // intermediate outputs alternate between two buffers
  void* level_out[KMAX];
  for (int j = 0; j < levels; ++j) level_out[j] = (char*)workspace + (j & 1) * one;
  return kpass_levels_forward(q, k, v, kg, grid, heads, out, batch, head_dim, dtype, scale, level_out, nullptr,
                              (hipStream_t)stream);
}

size_t squad_kpass_train_workspace_size(const int32_t grid[3], const int32_t* tiles, int32_t levels,
                                        int32_t heads, int32_t batch, int32_t head_dim, int32_t dtype) {
  KGeo kg;
  if (kpass_check(grid, tiles, levels, heads, batch, head_dim, dtype, kg)) return 0;
  return kpass_train_layout(kg, heads, batch, head_dim, dtype).total;
}

int squad_kpass_forward_train(const void* q, const void* k, const void* v, const int32_t grid[3],
                              const int32_t* tiles, int32_t levels, int32_t heads, void* out, int32_t batch,
                              int32_t head_dim, int32_t dtype, float scale, void* workspace,
                              size_t workspace_bytes, squad_stream_t stream) {
  KGeo kg;
  int st = kpass_check(grid, tiles, levels, heads, batch, head_dim, dtype, kg);
  if (st) return st;
  const size_t bytes = (size_t)heads * batch * kg.n * head_dim * elem_bytes(dtype);
  const void* in[3] = {q, k, v};
  st = check_ptrs(in, 3, out, bytes);
  if (st) return st;
  const KTrainLayout t = kpass_train_layout(kg, heads, batch, head_dim, dtype);
  if (!workspace || workspace_bytes < t.total) return SQUAD_ERR_WORKSPACE;
  if (misaligned(workspace)) return SQUAD_ERR_ALIGN;
  for (int i = 0; i < 3; ++i)
    if (overlap(in[i], bytes, workspace, t.total)) return SQUAD_ERR_ALIAS;
  if (overlap(out, bytes, workspace, t.total)) return SQUAD_ERR_ALIAS;
  if (!isfinite(scale)) return SQUAD_ERR_INVALID_ARG;
  char* ws = (char*)workspace;
  void* level_out[KMAX];
  for (int j = 0; j + 1 < levels; ++j) level_out[j] = ws + t.inter + (size_t)j * t.one_i;
  return kpass_levels_forward(q, k, v, kg, grid, heads, out, batch, head_dim, dtype, scale, level_out,
                              (float*)(ws + t.lse), (hipStream_t)stream);
}

int squad_kpass_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                         const int32_t grid[3], const int32_t* tiles, int32_t levels, int32_t heads, void* dq,
                         void* dk, void* dv, int32_t batch, int32_t head_dim, int32_t dtype, float scale,
                         void* workspace, size_t workspace_bytes, squad_stream_t stream) {
  KGeo kg;
  int st = kpass_check(grid, tiles, levels, heads, batch, head_dim, dtype, kg);
  if (st) return st;
  const size_t bytes = (size_t)heads * batch * kg.n * head_dim * elem_bytes(dtype);
  const void* in[5] = {q, k, v, out, dout};
  void* outs[3] = {dq, dk, dv};
  for (const void* p : in)
    if (!p) return SQUAD_ERR_INVALID_ARG;
  for (const void* p : outs)
    if (!p) return SQUAD_ERR_INVALID_ARG;
  if (!workspace) return SQUAD_ERR_WORKSPACE;
  for (const void* p : in)
    if (misaligned(p)) return SQUAD_ERR_ALIGN;
  for (const void* p : outs)
    if (misaligned(p)) return SQUAD_ERR_ALIGN;
  if (misaligned(workspace)) return SQUAD_ERR_ALIGN;
  const KTrainLayout t = kpass_train_layout(kg, heads, batch, head_dim, dtype);
  if (workspace_bytes < t.total) return SQUAD_ERR_WORKSPACE;
  for (int i = 0; i < 3; ++i) {
    for (const void* p : in)
      if (overlap(outs[i], bytes, p, bytes)) return SQUAD_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], bytes, outs[j], bytes)) return SQUAD_ERR_ALIAS;
    if (overlap(outs[i], bytes, workspace, t.total)) return SQUAD_ERR_ALIAS;
  }
  for (const void* p : in)
    if (overlap(p, bytes, workspace, t.total)) return SQUAD_ERR_ALIAS;
  if (!isfinite(scale)) return SQUAD_ERR_INVALID_ARG;

  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  const bool bf16 = dtype == SQUAD_DTYPE_BF16;
  const size_t rows = (size_t)heads * batch * kg.n;
  const bool parts = bf16;   // the fp16 part hand-off between the levels
  float* dq_acc = parts ? nullptr : bf16 ? (float*)(ws + t.dq_acc) : (float*)dq;
  float* dk_acc = parts ? nullptr : bf16 ? (float*)(ws + t.dk_acc) : (float*)dk;
  float* dq_sc = parts ? (float*)(ws + t.dq_sc) : nullptr;
  float* dk_sc = parts ? (float*)(ws + t.dk_sc) : nullptr;
  auto inter = [&](int j) -> void* { return ws + t.inter + (size_t)(j - 1) * t.one_i; };   // o_j, j >= 1
  // from the last level down: level j's values are o_j (v for j = 0), its output
  // o_(j+1) (out for the last), its upstream gradient that of o_(j+1) (dout for
  // the last); it adds its parts of dq and dk and writes the gradient of o_j
  for (int j = levels - 1; j >= 0; --j) {
    const void* vals = j == 0 ? v : inter(j);
    const void* outj = j == levels - 1 ? out : inter(j + 1);
    const void* up = j == levels - 1 ? dout : ws + t.dgrad[(j + 1) & 1];
    void* dvj = j == 0 ? dv : ws + t.dgrad[j & 1];
    const uint32_t mode = parts ? (j == levels - 1 ? kPartWrite : (j == 0 ? kPartFinal : kPartAdd))
                                : j == levels - 1 ? kAccWrite : (j == 0 ? kAccFinal : kAccAdd);
    auto fill = [&](auto& a) {
      kpass_bwd_common(a, kg, j, heads, batch, head_dim, scale);
      a.q = q; a.k = k; a.v = vals; a.o = outj; a.dout = up;
      a.mv = a.mqk; a.mo = a.mqk; a.mdo = a.mqk; a.mdq = a.mqk; a.mdk = a.mqk; a.mdv = a.mqk;
      a.lse = (const float*)(ws + t.lse) + (size_t)j * rows;
      a.dsum = (float*)(ws + t.dsum);
      a.dq = dq; a.dk = dk; a.dq_acc = dq_acc; a.dk_acc = dk_acc; a.dv = dvj;
      a.dq_sc = dq_sc; a.dk_sc = dk_sc;
      a.final_pass = mode;
    };
    if (j == 0 || j == levels - 1) {
      BwdArgs a;
      memset(&a, 0, sizeof(a));
      st = kpass_end_map(kg, grid, j, heads, head_dim, a.mqk);
      if (st) return st;
      fill(a);
      st = run_bwd(a, head_dim, dtype, BwdTypes{j >= 1, j < levels - 1}, s);
    } else {
      BwdArgsK a;
      memset(&a, 0, sizeof(a));
      a.mqk = kpass_map(kg, j, heads, head_dim);
      fill(a);
      if (a.units == 0) continue;
      if (bf16 && bwd_bf16_fused(a.L, false)) {
        st = launch_bwd_bf16_small_k(a, head_dim, s) == hipSuccess ? SQUAD_OK : SQUAD_ERR_HIP;
      } else {
        for (int kind = 0; kind < 2 && !st; ++kind) {
          const hipError_t e = bf16 ? launch_bwd_bf16_k(a, head_dim, kind == 1, s)
                                    : launch_bwd_f32_k(a, head_dim, kind == 1, s);
          st = e == hipSuccess ? SQUAD_OK : SQUAD_ERR_HIP;
        }
      }
    }
    if (st) return st;
  }
  return SQUAD_OK;
}

int squad_debug_kpass_offsets(const int32_t grid[3], const int32_t* tiles, int32_t levels, int32_t level,
                              int32_t heads, int32_t batch, int32_t head_dim, int64_t* offsets) {
  KGeo kg;
  int st = make_kgeo(grid, tiles, levels, kg);
  if (st) return st;
  if (level < 0 || level >= levels || !offsets || heads <= 0 || batch <= 0 || head_dim <= 0)
    return SQUAD_ERR_INVALID_ARG;
  const RowMapK m = kpass_map(kg, level, heads, head_dim);
  const uint32_t L = (uint32_t)kpass_rows(kg, level);
  const uint32_t U = (uint32_t)(kg.n / L);
  size_t i = 0;
  for (uint32_t b = 0; b < (uint32_t)batch; ++b)
    for (uint32_t h = 0; h < (uint32_t)heads; ++h)
      for (uint32_t s = 0; s < U; ++s) {
        const int64_t base = m.base(b, h, s);
        for (uint32_t r = 0; r < L; ++r) offsets[i++] = base + m.row_off(r);
      }
  return SQUAD_OK;
}

}  // extern "C"

// ---- the block around the operator: fused QKV projection, attention, output
// projection (plain GEMMs on rocBLAS; the attention reads q, k, v straight out of
// the projection's output rows)
namespace {

// y[M, N] = x[M, K] w[N, K]^T, all row-major (rocBLAS is column-major: y^T = w x^T)
int gemm_xwt(rocblas_handle hnd, const void* x, const void* w, void* y, int64_t M, int64_t N, int64_t K,
             int32_t dtype) {
  const float one = 1.f, zero = 0.f;
  const rocblas_datatype t = dtype == SQUAD_DTYPE_BF16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
  const rocblas_status st = rocblas_gemm_ex(hnd, rocblas_operation_transpose, rocblas_operation_none,
                                            (rocblas_int)N, (rocblas_int)M, (rocblas_int)K, &one, w, t,
                                            (rocblas_int)K, x, t, (rocblas_int)K, &zero, y, t, (rocblas_int)N, y,
                                            t, (rocblas_int)N, rocblas_datatype_f32_r, rocblas_gemm_algo_standard,
                                            0, 0);
  return st == rocblas_status_success ? SQUAD_OK : SQUAD_ERR_HIP;
}

struct BlockLayout {
  size_t qkv, ws, attn, total;
};

int block_layout(const Geo& g, int32_t heads, int32_t batch, int32_t head_dim, int32_t dtype, BlockLayout& b) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t esz = elem_bytes(dtype);
  const size_t rows = (size_t)batch * (size_t)g.n;
  const size_t hidden = (size_t)heads * head_dim;
  size_t bytes = 0, wbytes = 0;
  Geo g2;
  const int32_t grid[3] = {(int32_t)g.T, (int32_t)g.H, (int32_t)g.W};
  const int32_t tile[3] = {(int32_t)g.tt, (int32_t)g.th, (int32_t)g.tw};
  int st = check_grid_call(grid, tile, heads, batch, head_dim, dtype, g2, bytes, &wbytes, true);
  if (st) return st;
  b.qkv = 0;
  b.ws = al(rows * 3 * hidden * esz);
  b.attn = al(b.ws + wbytes);
  b.total = al(b.attn + rows * hidden * esz);
  return SQUAD_OK;
}

// q, k, v of the block are slices of the projection's rows (stride 3 * hidden):
// the maps' row unit covers that span too.
int block_row_unit(Geo& g, int32_t heads, int32_t head_dim) {
  const uint64_t hidden = (uint64_t)heads * (uint64_t)head_dim;
  const uint64_t cells = (uint64_t)g.G * (uint64_t)g.Wn;
  return pick_row_unit(g, std::max(cells * hidden, (uint64_t)g.n * 3 * hidden), head_dim);
}

}  // namespace

extern "C" {

int squad_blas_create(squad_blas_t* handle) {
  if (!handle) return SQUAD_ERR_INVALID_ARG;
  rocblas_handle h = nullptr;
  if (rocblas_create_handle(&h) != rocblas_status_success || !h) return SQUAD_ERR_HIP;
  *handle = (squad_blas_t)h;
  return SQUAD_OK;
}

int squad_blas_destroy(squad_blas_t handle) {
  if (!handle) return SQUAD_ERR_INVALID_ARG;
  return rocblas_destroy_handle((rocblas_handle)handle) == rocblas_status_success ? SQUAD_OK : SQUAD_ERR_HIP;
}

size_t squad_block_workspace_size(const int32_t grid[3], const int32_t tile[3], int32_t heads, int32_t batch,
                                  int32_t head_dim, int32_t dtype) {
  Geo g;
  size_t bytes = 0;
  if (check_grid_call(grid, tile, heads, batch, head_dim, dtype, g, bytes, nullptr, true)) return 0;
  BlockLayout b;
  if (block_layout(g, heads, batch, head_dim, dtype, b)) return 0;
  if (block_row_unit(g, heads, head_dim)) return 0;   // as squad_block_forward
  return b.total;
}

int squad_block_forward(const void* x, const void* w_qkv, const void* w_out, const int32_t grid[3],
                        const int32_t tile[3], int32_t heads, void* y, int32_t batch, int32_t head_dim,
                        int32_t dtype, float scale, int32_t dense, squad_blas_t blas, void* workspace,
                        size_t workspace_bytes, squad_stream_t stream) {
  Geo g;
  size_t bytes = 0;
  int st = check_grid_call(grid, tile, heads, batch, head_dim, dtype, g, bytes, nullptr, true);
  if (st) return st;
  if (dense != 0 && dense != 1) return SQUAD_ERR_INVALID_ARG;
  BlockLayout lay;
  st = block_layout(g, heads, batch, head_dim, dtype, lay);
  if (st) return st;
  const int64_t hidden = (int64_t)heads * head_dim;
  st = block_row_unit(g, heads, head_dim);
  if (st) return st;
  // the dense comparator takes narrow maps only
  if (dense && g.ru > 1) return SQUAD_ERR_SHAPE;
  if ((int64_t)batch * g.n >= (int64_t(1) << 31) || 3 * hidden >= (int64_t(1) << 31)) return SQUAD_ERR_SHAPE;
  const size_t wq_bytes = (size_t)3 * hidden * hidden * elem_bytes(dtype);
  const size_t wo_bytes = (size_t)hidden * hidden * elem_bytes(dtype);
  if (!x || !w_qkv || !w_out || !y || !blas) return SQUAD_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < lay.total) return SQUAD_ERR_WORKSPACE;
  if (misaligned(x) || misaligned(w_qkv) || misaligned(w_out) || misaligned(y) || misaligned(workspace))
    return SQUAD_ERR_ALIGN;
  if (overlap(y, bytes, x, bytes) || overlap(y, bytes, w_qkv, wq_bytes) || overlap(y, bytes, w_out, wo_bytes) ||
      overlap(y, bytes, workspace, lay.total) || overlap(x, bytes, workspace, lay.total) ||
      overlap(w_qkv, wq_bytes, workspace, lay.total) || overlap(w_out, wo_bytes, workspace, lay.total))
    return SQUAD_ERR_ALIAS;
  if (!isfinite(scale)) return SQUAD_ERR_INVALID_ARG;

  rocblas_handle hnd = (rocblas_handle)blas;
  hipStream_t s = (hipStream_t)stream;
  if (rocblas_set_stream(hnd, s) != rocblas_status_success) return SQUAD_ERR_HIP;

  char* ws = (char*)workspace;
  const size_t esz = elem_bytes(dtype);
  const int64_t M = (int64_t)batch * g.n;
  char* qkv = ws + lay.qkv;
  char* attn = ws + lay.attn;
  st = gemm_xwt(hnd, x, w_qkv, qkv, M, 3 * hidden, hidden, dtype);
  if (st) return st;
  const char* q = qkv;
  const char* k = qkv + hidden * esz;
  const char* v = qkv + 2 * hidden * esz;
  if (dense) {
    // comparator: full softmax attention over all n tokens, same projections
    AttnArgs a = attn_args(q, k, v, attn, (uint32_t)g.n, 1, heads, batch, head_dim, scale);
    RowMap m;
    m.sB = g.n * 3 * hidden;
    m.sH = head_dim;
    m.unit = linear(0);
    m.row = linear32(3 * hidden);
    a.mqk = m; a.mv = m;
    a.mo = m;
    a.mo.sB = g.n * hidden;
    a.mo.row = linear32(hidden);
    st = run_attn(a, head_dim, dtype, s);
  } else {
    st = forward_local(q, k, v, g, heads, batch, head_dim, dtype, scale, ws + lay.ws, s, nullptr, 3 * hidden);
    if (!st)
      st = forward_global(q, k, attn, g, heads, batch, head_dim, dtype, scale, ws + lay.ws, s, nullptr,
                          3 * hidden);
  }
  if (st) return st;
  return gemm_xwt(hnd, attn, w_out, y, M, hidden, hidden, dtype);
}

// ---- the forward for callers that cannot allocate (graph capture, serving loops):
// its local output lives in a file-scope device array instead of a caller's
// workspace.  Each device holds its own copy until the process ends; host code
// uses the address hipGetSymbolAddress gives for the current device, never the
// array's name (a host-side stand-in).
static __device__ __align__(256) unsigned char scratch[SQUAD_NOALLOC_SCRATCH_BYTES];

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];   // per device: the device address of `scratch`

// The current device's copy of `scratch`, looked up once per device (with that
// device current) and kept.
int scratch_address(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SQUAD_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SQUAD_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return SQUAD_OK;
}

}  // namespace

extern "C" {

int squad_attn_forward_noalloc(const void* q, const void* k, const void* v, const int32_t grid[3],
                               const int32_t tile[3], int32_t heads, void* out, int32_t batch,
                               int32_t head_dim, int32_t dtype, float scale, squad_stream_t stream) {
  Geo g;
  size_t bytes = 0;
  int st = check_grid_call(grid, tile, heads, batch, head_dim, dtype, g, bytes, nullptr, true);
  if (st) return st;
  const void* in[3] = {q, k, v};
  st = check_ptrs(in, 3, out, bytes);
  if (st) return st;
  if (!isfinite(scale)) return SQUAD_ERR_INVALID_ARG;
  const size_t esz = elem_bytes(dtype);
  // the local output of one (batch, head): G * Wn rows of head_dim elements
  const size_t per_head = (size_t)g.G * (size_t)g.Wn * (size_t)head_dim * esz;
  if (per_head > SQUAD_NOALLOC_SCRATCH_BYTES) return SQUAD_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  if ((size_t)batch * (size_t)heads * per_head <= SQUAD_NOALLOC_SCRATCH_BYTES) {
    st = forward_local(q, k, v, g, heads, batch, head_dim, dtype, scale, ws, s);
    if (st) return st;
    return forward_global(q, k, out, g, heads, batch, head_dim, dtype, scale, ws, s);
  }
  // slices of at most `hs` heads of one batch element, one after the other on the
  // stream (each slice's global pass has read the scratch before the next local
  // pass writes it); the token maps keep the full row stride heads * head_dim
  const int64_t ts = (int64_t)heads * head_dim;
  const int32_t hs = (int32_t)std::min<size_t>(SQUAD_NOALLOC_SCRATCH_BYTES / per_head, (size_t)heads);
  for (int32_t b = 0; b < batch; ++b)
    for (int32_t h0 = 0; h0 < heads; h0 += hs) {
      const int32_t hn = std::min(hs, heads - h0);
      const size_t off = ((size_t)b * (size_t)g.n * (size_t)ts + (size_t)h0 * (size_t)head_dim) * esz;
      const char* qs = (const char*)q + off;
      const char* ks = (const char*)k + off;
      st = forward_local(qs, ks, (const char*)v + off, g, hn, 1, head_dim, dtype, scale, ws, s, nullptr, ts);
      if (st) return st;
      st = forward_global(qs, ks, (char*)out + off, g, hn, 1, head_dim, dtype, scale, ws, s, nullptr, ts, ts);
      if (st) return st;
    }
  return SQUAD_OK;
}

int squad_debug_mfma_probe(float* out, int32_t blocks, int32_t iters, squad_stream_t stream) {
  if (!out || blocks <= 0 || iters <= 0) return SQUAD_ERR_INVALID_ARG;
  if (misaligned(out)) return SQUAD_ERR_ALIGN;
  return launch_mfma_probe(out, blocks, iters, (hipStream_t)stream) == hipSuccess ? SQUAD_OK : SQUAD_ERR_HIP;
}

}  // extern "C"
