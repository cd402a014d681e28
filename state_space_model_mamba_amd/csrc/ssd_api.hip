// C ABI of libssd_bwd.so (declared in include/ssd_bwd.h): argument checks,
// the workspace layout and the launch sequence of the SSD backward.
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <set>
#include <utility>

#include "ssd_bwd.h"
#include "ssd_problem.h"

namespace ssd {

hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes) {
  static std::mutex mu;
  static std::set<std::pair<int, const void*>> done;   // (device, kernel) already raised
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({dev, kernel})) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
  if (e == hipSuccess) done.insert({dev, kernel});
  return e;
}

namespace {
std::atomic<int> g_head_blocks{0}, g_fwd_heads{0}, g_group_path{0};
}  // namespace

int head_blocks_override() { return g_head_blocks.load(std::memory_order_relaxed); }
int fwd_heads_per_block_override() { return g_fwd_heads.load(std::memory_order_relaxed); }
int group_path_override() { return g_group_path.load(std::memory_order_relaxed); }

}  // namespace ssd

extern "C" int ssd_set_group_path(int path) {
  if (path < 0 || path > 2) return SSD_ERR_INVALID_ARG;
  ssd::g_group_path.store(path, std::memory_order_relaxed);
  return SSD_OK;
}

extern "C" int ssd_set_launch_geometry(int head_blocks, int fwd_heads_per_block) {
  if (head_blocks < 0 || fwd_heads_per_block < 0) return SSD_ERR_INVALID_ARG;
  ssd::g_head_blocks.store(head_blocks, std::memory_order_relaxed);
  ssd::g_fwd_heads.store(fwd_heads_per_block, std::memory_order_relaxed);
  return SSD_OK;
}

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t segpos, cinfo, acs, dtc, dfe, hin, dstate, dcb, dcbt, dcbp, dcp, dbp, cbt, offd, endd, slot_dA, slot_dD,
      slot_dDp, slot_ddtb, seqstart, total;
  int nc, ntg, nslice, nslice_bd;
  bool fused;
};

bool is_bf16(const ssd_shape* s) { return s->io_dtype == SSD_IO_BF16; }

// head slices of the split path's k_dc / k_db: doubled while their grid (one
// block per (batch, group, chunk, widest dstate tile, slice)) has fewer than
// 256 blocks and a slice keeps at least one head
int split_slices_bd(const ssd_shape* s) {
  const int64_t nc = (s->seqlen + s->chunk_size - 1) / s->chunk_size;
  const int64_t hpg = s->nheads / s->ngroups;
  const int64_t tiles = s->batch * s->ngroups * nc * (s->dstate / ssd::group_ntile(static_cast<int>(s->dstate), is_bf16(s)));
  int S = 1;
  while (tiles * S < 256 && 2 * S <= hpg) S *= 2;
  return S;
}

// dstate tile of the split path's k_dc / k_db: the widest that divides N,
// halved (down to 32 columns) while that grid, with its head slices, has
// fewer than 256 blocks
int split_ntile(const ssd_shape* s) {
  const int N = static_cast<int>(s->dstate);
  int nt = ssd::group_ntile(N, is_bf16(s));
  const int64_t nc = (s->seqlen + s->chunk_size - 1) / s->chunk_size;
  const int64_t S = split_slices_bd(s);
  while (nt > 32 && N % (nt / 2) == 0 && s->batch * s->ngroups * nc * (N / nt) * S < 256) nt /= 2;
  return nt;
}

// head slices of the split path's k_dcb: doubled while its grid has fewer
// than 256 blocks and a slice keeps at least one head
int split_slices(const ssd_shape* s) {
  const int64_t nc = (s->seqlen + s->chunk_size - 1) / s->chunk_size;
  const int64_t hpg = s->nheads / s->ngroups;
  int S = 1;
  while (s->batch * s->ngroups * nc * S < 256 && 2 * S <= hpg) S *= 2;
  return S;
}

// The group stage (dCB, dC, dB) runs split (k_dcb, k_dc, k_db: one block per
// (batch, group, chunk, dstate tile of k_dc / k_db)) when that grid has at
// least 256 blocks, one per CU of an MI355X.  Below that it runs fused
// (k_cb, k_grp, whose 64-row slabs multiply the blocks by Q / 64) when a
// group has at most 16 heads; with more heads per group, every fused block
// walks them all, and the split path, with its kernels' heads cut into
// slices, is faster (measured: 7 packed sequences of 16384 rows, 64 heads in
// one group, group stage 0.48 against 0.85 ms; 2048 rows, 8 groups of 16
// heads, fused 0.11 against 0.13 ms).  A function of the shape
// only (or the test override); the two paths add the same terms in different
// orders, so their results agree to rounding, not bit for bit.
bool group_fused(const ssd_shape* s) {
  const int ov = ssd::group_path_override();
  if (ov == 1) return true;
  if (ov == 2) return false;
  const int64_t nc = (s->seqlen + s->chunk_size - 1) / s->chunk_size;
  const int64_t ntg = s->dstate / ssd::group_ntile(static_cast<int>(s->dstate), is_bf16(s));
  return s->batch * s->ngroups * nc * ntg < 256 && s->nheads / s->ngroups <= 16;
}

int check_shape(const ssd_shape* s) {
  if (!s) return SSD_ERR_INVALID_ARG;
  if (s->batch < 1 || s->seqlen < 1 || s->nheads < 1 || s->headdim < 1 || s->ngroups < 1 ||
      s->dstate < 1 || s->chunk_size < 1 || s->nseqs < 0 || s->reserved != 0)
    return SSD_ERR_INVALID_ARG;
  if (s->io_dtype != SSD_IO_BF16 && s->io_dtype != SSD_IO_F32) return SSD_ERR_INVALID_ARG;
  if (s->nheads % s->ngroups) return SSD_ERR_UNSUPPORTED_SHAPE;
  const int64_t Q = s->chunk_size, P = s->headdim, N = s->dstate;
  // dstate slabs are 32 (bf16) or 16 (fp32) columns wide
  if (N % (is_bf16(s) ? 32 : 16) || N > 256) return SSD_ERR_UNSUPPORTED_SHAPE;
  if (ssd::head_lds_bytes(static_cast<int>(Q), static_cast<int>(P), is_bf16(s)) == ~size_t(0))
    return SSD_ERR_UNSUPPORTED_SHAPE;
  // index arithmetic inside the kernels uses int for positions and block counts
  const int64_t nc = (s->seqlen + Q - 1) / Q;
  if (s->seqlen > (int64_t(1) << 30) || s->batch * s->nheads * nc > (int64_t(1) << 30) ||
      s->nheads > (1 << 20) || s->batch > (1 << 20) || s->nseqs > (int64_t(1) << 30))
    return SSD_ERR_UNSUPPORTED_SHAPE;
  // the rows of one chunk of x / dy (all heads) and of B / C (all groups) are
  // addressed with 32-bit byte offsets from the chunk's first row
  const int64_t esize = is_bf16(s) ? 2 : 4;
  if (Q * s->nheads * P * esize > (int64_t(1) << 31) || Q * s->ngroups * N * esize > (int64_t(1) << 31))
    return SSD_ERR_UNSUPPORTED_SHAPE;
  const size_t lim = 160 * 1024;
  const bool fused = group_fused(s);
  const size_t group_lds =
      fused ? ssd::grp_lds_bytes(static_cast<int>(Q), static_cast<int>(P),
                                 ssd::grp_ntile(static_cast<int>(N), is_bf16(s)), is_bf16(s))
            : std::max(ssd::dcb_lds_bytes(static_cast<int>(Q), static_cast<int>(P), is_bf16(s)),
                       ssd::dbdc_lds_bytes(static_cast<int>(Q), static_cast<int>(P), split_ntile(s), is_bf16(s)));
  if (ssd::head_lds_bytes(static_cast<int>(Q), static_cast<int>(P), is_bf16(s)) > lim || group_lds > lim ||
      ssd::fwd_lds_bytes(static_cast<int>(Q), static_cast<int>(P), is_bf16(s)) > lim)
    return SSD_ERR_UNSUPPORTED_SHAPE;
  return SSD_OK;
}

Layout make_layout(const ssd_shape* s) {
  Layout L;
  const size_t B = s->batch, H = s->nheads, Q = s->chunk_size, P = s->headdim, N = s->dstate;
  const size_t nc = (s->seqlen + s->chunk_size - 1) / s->chunk_size;
  L.fused = group_fused(s);
  const size_t ntg = N / (L.fused ? ssd::grp_ntile(static_cast<int>(N), is_bf16(s)) : split_ntile(s));
  L.nslice = L.fused ? 1 : split_slices(s);
  L.nslice_bd = L.fused ? 1 : split_slices_bd(s);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.segpos = take(B * nc * Q * 4);
  L.cinfo = take(B * nc * ssd::CINFO * 4);
  L.acs = take(B * H * nc * Q * 4);
  L.dtc = take(B * H * nc * Q * 4);
  L.dfe = take(B * H * nc * Q * 4);
  const size_t es = is_bf16(s) ? 2 : 4;
  L.hin = take(B * H * nc * P * N * es);
  L.dstate = take(B * H * nc * P * N * es);
  const size_t dcb_bytes = L.fused ? 0 : B * s->ngroups * nc * Q * Q * es;
  L.dcb = take(dcb_bytes);
  L.dcbt = take(dcb_bytes);
  L.dcbp = take(L.nslice > 1 ? B * s->ngroups * nc * L.nslice * (Q * (Q + 16) / 2) * 4 : 0);
  const size_t bd_bytes = L.nslice_bd > 1 ? B * s->ngroups * nc * L.nslice_bd * Q * N * 4 : 0;
  L.dcp = take(bd_bytes);
  L.dbp = take(bd_bytes);
  L.cbt = take(B * s->ngroups * nc * (Q * (Q + 16) / 2) * 4);
  L.offd = take(B * H * nc * ntg * Q * 4);
  L.endd = take(B * H * nc * ntg * 4);
  L.slot_dA = take(B * nc * H * 4);
  L.slot_dD = take(B * nc * H * 4);
  L.slot_ddtb = take(B * nc * H * 4);
  L.slot_dDp = take(B * nc * H * P * 4);
  L.seqstart = take((s->nseqs > 0 ? s->nseqs : 1) * 4);
  L.total = off;
  L.nc = static_cast<int>(nc);
  L.ntg = static_cast<int>(ntg);
  return L;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int ssd_bwd_workspace_size(const ssd_shape* shape, size_t* bytes) {
  const int rc = check_shape(shape);
  if (rc) return rc;
  if (!bytes) return SSD_ERR_INVALID_ARG;
  *bytes = make_layout(shape).total;
  return SSD_OK;
}

extern "C" int ssd_bwd_workspace_region(const ssd_shape* shape, int region, size_t* offset, size_t* bytes) {
  const int rc = check_shape(shape);
  if (rc) return rc;
  if (!offset || !bytes) return SSD_ERR_INVALID_ARG;
  const Layout L = make_layout(shape);
  const size_t B = shape->batch, H = shape->nheads, Q = shape->chunk_size, P = shape->headdim,
               N = shape->dstate, nc = L.nc;
  switch (region) {
    case SSD_WS_ACS: *offset = L.acs; *bytes = B * H * nc * Q * 4; return SSD_OK;
    case SSD_WS_HIN: *offset = L.hin; *bytes = B * H * nc * P * N * (is_bf16(shape) ? 2 : 4); return SSD_OK;
    case SSD_WS_DSTATE: *offset = L.dstate; *bytes = B * H * nc * P * N * (is_bf16(shape) ? 2 : 4); return SSD_OK;
    default: return SSD_ERR_INVALID_ARG;
  }
}

extern "C" const char* ssd_status_string(int status) {
  switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_INVALID_ARG: return "invalid argument";
    case SSD_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case SSD_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SSD_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case SSD_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

extern "C" int ssd_bwd_version(void) { return (1 << 16) | 0; }

namespace {

const char* const kStageNames[] = {"prep", "state_fwd", "state_bwd", "dcb", "dbdc", "head_bwd", "reduce"};
constexpr int kStages = 7;

// Shape and workspace fields of the kernels' problem descriptor.
void fill_problem(const ssd_shape* shape, const Layout& L, void* workspace, ssd::Problem& pb) {
  memset(&pb, 0, sizeof(pb));
  pb.B = static_cast<int>(shape->batch);
  pb.L = static_cast<int>(shape->seqlen);
  pb.H = static_cast<int>(shape->nheads);
  pb.P = static_cast<int>(shape->headdim);
  pb.G = static_cast<int>(shape->ngroups);
  pb.N = static_cast<int>(shape->dstate);
  pb.Q = static_cast<int>(shape->chunk_size);
  pb.nc = L.nc;
  pb.hpg = pb.H / pb.G;
  pb.nseqs = shape->nseqs > 0 ? static_cast<int>(shape->nseqs) : 1;
  pb.ntg = L.ntg;
  char* ws = static_cast<char*>(workspace);
  pb.segpos = reinterpret_cast<int32_t*>(ws + L.segpos);
  pb.cinfo = reinterpret_cast<int32_t*>(ws + L.cinfo);
  pb.acs = reinterpret_cast<float*>(ws + L.acs);
  pb.dtc = reinterpret_cast<float*>(ws + L.dtc);
  pb.dfe = reinterpret_cast<float*>(ws + L.dfe);
  pb.hin = ws + L.hin;
  pb.dstate = ws + L.dstate;
  pb.dcb = ws + L.dcb;
  pb.dcbt = ws + L.dcbt;
  pb.nslice = L.nslice;
  pb.dcbp = reinterpret_cast<float*>(ws + L.dcbp);
  pb.nslice_bd = L.nslice_bd;
  pb.dcp = reinterpret_cast<float*>(ws + L.dcp);
  pb.dbp = reinterpret_cast<float*>(ws + L.dbp);
  pb.cbt = reinterpret_cast<float*>(ws + L.cbt);
  pb.offd = reinterpret_cast<float*>(ws + L.offd);
  pb.endd = reinterpret_cast<float*>(ws + L.endd);
  pb.slot_dA = reinterpret_cast<float*>(ws + L.slot_dA);
  pb.slot_dD = reinterpret_cast<float*>(ws + L.slot_dD);
  pb.slot_ddtb = reinterpret_cast<float*>(ws + L.slot_ddtb);
  pb.slot_dDp = reinterpret_cast<float*>(ws + L.slot_dDp);
  pb.seqstart = reinterpret_cast<int32_t*>(ws + L.seqstart);
}

// The options' fields of the problem (fe NULL: none).
int fill_frontend(const ssd_options* fe, ssd::Problem& pb) {
  pb.fe = 0;
  pb.d_hp = 0;
  pb.dt_bias = nullptr;
  pb.dt_softplus = 0;
  pb.dt_min = -__builtin_inff();
  pb.dt_max = __builtin_inff();
  pb.dlast = nullptr;
  if (!fe) return SSD_OK;
  if (!(fe->dt_min <= fe->dt_max)) return SSD_ERR_INVALID_ARG;   // (also rejects NaN)
  if (fe->dt_bias && !aligned16(fe->dt_bias)) return SSD_ERR_MISALIGNED;
  pb.dt_bias = fe->dt_bias;
  pb.dt_softplus = fe->dt_softplus != 0;
  pb.dt_min = fe->dt_min;
  pb.dt_max = fe->dt_max;
  pb.fe = pb.dt_bias || pb.dt_softplus || pb.dt_min > -__builtin_inff() || pb.dt_max < __builtin_inff();
  pb.d_hp = fe->d_per_channel != 0;
  pb.dlast = fe->d_last_states;
  return SSD_OK;
}

int run_bwd(const ssd_shape* shape, const ssd_options* fe, const void* x, const float* dt, const float* A,
            const void* B, const void* C, const float* D, const void* z, const void* dy,
            const float* initial_states, const int32_t* seq_idx, void* dx, float* ddt, float* dA, void* dB,
            void* dC, float* dD, float* d_initial_states, float* ddt_bias, void* dz, void* workspace,
            size_t workspace_bytes, void* stream, void* const* events) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (ddt_bias && !(fe && fe->dt_bias)) return SSD_ERR_INVALID_ARG;
  if ((z != nullptr) != (dz != nullptr)) return SSD_ERR_INVALID_ARG;
  if (z && (z == dx || dz == dx || dz == dy)) return SSD_ERR_INVALID_ARG;   // dx holds the gated dy
  if (const void* yp = fe ? fe->y_pre_gate : nullptr) {
    if (!aligned16(yp)) return SSD_ERR_MISALIGNED;
    if (yp == dx || yp == dz || yp == dy || yp == z || yp == x) return SSD_ERR_INVALID_ARG;
  }
  for (const void* p : {static_cast<const void*>(ddt_bias), z, static_cast<const void*>(dz)})
    if (p && !aligned16(p)) return SSD_ERR_MISALIGNED;
  if (!x || !dt || !A || !B || !C || !dy || !dx || !ddt || !dA || !dB || !dC || !workspace)
    return SSD_ERR_INVALID_ARG;
  if (dD && !D) return SSD_ERR_INVALID_ARG;
  if (!seq_idx && (initial_states || d_initial_states) && shape->nseqs != shape->batch)
    return SSD_ERR_INVALID_ARG;
  if ((initial_states || d_initial_states) && shape->nseqs < 1) return SSD_ERR_INVALID_ARG;
  const void* ptrs[] = {x, dt, A, B, C, D, dy, initial_states, seq_idx, dx, ddt, dA, dB, dC, dD,
                        d_initial_states, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSD_ERR_MISALIGNED;
  if (events)
    for (int i = 0; i <= kStages; ++i)
      if (!events[i]) return SSD_ERR_INVALID_ARG;
  const Layout L = make_layout(shape);
  if (workspace_bytes < L.total) return SSD_ERR_WORKSPACE_TOO_SMALL;

  ssd::Problem pb;
  fill_problem(shape, L, workspace, pb);
  if ((rc = fill_frontend(fe, pb))) return rc;
  pb.x = x; pb.dt = dt; pb.A = A; pb.Bm = B; pb.Cm = C; pb.D = D; pb.dy = dy;
  pb.h0 = initial_states; pb.seq_idx = seq_idx;
  pb.dx = dx; pb.ddt = ddt; pb.dA = dA; pb.dB = dB; pb.dC = dC; pb.dD = dD;
  pb.dinit = d_initial_states;
  pb.ddt_bias = ddt_bias;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = is_bf16(shape);
  auto mark = [&](int i) -> bool {
    return !events || hipEventRecord(static_cast<hipEvent_t>(events[i]), s) == hipSuccess;
  };
  if (!mark(0)) return SSD_ERR_HIP;
  if (ssd::launch_prep(pb, s) != hipSuccess || !mark(1)) return SSD_ERR_HIP;
  if (ssd::launch_state_fwd(pb, bf16, s) != hipSuccess || !mark(2)) return SSD_ERR_HIP;
  if (z) {
    // gate pass: the gated dy into dx's place and dz, with y recomputed, or
    // read from the forward's saved copy in one elementwise pass; the stages
    // below read dy from there
    ssd::Problem pg = pb;
    pg.z = z; pg.dout = dy; pg.dz = dz; pg.y = dx;
    pg.ypre = fe ? fe->y_pre_gate : nullptr;
    if ((pg.ypre ? ssd::launch_gate_bwd(pg, bf16, s) : ssd::launch_fwd_out(pg, bf16, s)) != hipSuccess)
      return SSD_ERR_HIP;
    pb.dy = dx;
  }
  if (ssd::launch_state_bwd(pb, bf16, s) != hipSuccess || !mark(3)) return SSD_ERR_HIP;
  if ((L.fused ? ssd::launch_cb(pb, bf16, s) : ssd::launch_dcb(pb, bf16, s)) != hipSuccess || !mark(4))
    return SSD_ERR_HIP;
  if ((L.fused ? ssd::launch_grp(pb, bf16, s) : ssd::launch_dbdc(pb, bf16, s)) != hipSuccess || !mark(5))
    return SSD_ERR_HIP;
  if (ssd::launch_head_bwd(pb, bf16, s) != hipSuccess || !mark(6)) return SSD_ERR_HIP;
  if (ssd::launch_reduce(pb, s) != hipSuccess || !mark(7)) return SSD_ERR_HIP;
  return SSD_OK;
}

}  // namespace

extern "C" int ssd_bwd(const ssd_shape* shape, const void* x, const float* dt, const float* A,
                       const void* B, const void* C, const float* D, const void* dy,
                       const float* initial_states, const int32_t* seq_idx, void* dx, float* ddt,
                       float* dA, void* dB, void* dC, float* dD, float* d_initial_states,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return run_bwd(shape, nullptr, x, dt, A, B, C, D, nullptr, dy, initial_states, seq_idx, dx, ddt, dA, dB, dC,
                 dD, d_initial_states, nullptr, nullptr, workspace, workspace_bytes, stream, nullptr);
}

extern "C" int ssd_bwd_ex(const ssd_shape* shape, const ssd_options* fe, const void* x, const float* dt,
                          const float* A, const void* B, const void* C, const float* D, const void* z,
                          const void* dy, const float* initial_states, const int32_t* seq_idx, void* dx,
                          float* ddt, float* dA, void* dB, void* dC, float* dD, float* d_initial_states,
                          float* ddt_bias, void* dz, void* workspace, size_t workspace_bytes, void* stream) {
  return run_bwd(shape, fe, x, dt, A, B, C, D, z, dy, initial_states, seq_idx, dx, ddt, dA, dB, dC, dD,
                 d_initial_states, ddt_bias, dz, workspace, workspace_bytes, stream, nullptr);
}

extern "C" int ssd_bwd_profiled(const ssd_shape* shape, const void* x, const float* dt, const float* A,
                                const void* B, const void* C, const float* D, const void* dy,
                                const float* initial_states, const int32_t* seq_idx, void* dx,
                                float* ddt, float* dA, void* dB, void* dC, float* dD,
                                float* d_initial_states, void* workspace, size_t workspace_bytes,
                                void* stream, void* const* events) {
  if (!events) return SSD_ERR_INVALID_ARG;
  return run_bwd(shape, nullptr, x, dt, A, B, C, D, nullptr, dy, initial_states, seq_idx, dx, ddt, dA, dB, dC,
                 dD, d_initial_states, nullptr, nullptr, workspace, workspace_bytes, stream, events);
}

namespace {

int run_fwd(const ssd_shape* shape, const ssd_options* fe, const void* x, const float* dt, const float* A,
            const void* B, const void* C, const float* D, const void* z, const float* initial_states,
            const int32_t* seq_idx, void* y, float* final_states, void* workspace, size_t workspace_bytes,
            void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (z && !aligned16(z)) return SSD_ERR_MISALIGNED;
  if (!x || !dt || !A || !B || !C || !y || !workspace) return SSD_ERR_INVALID_ARG;
  if (const void* yp = fe ? fe->y_pre_gate : nullptr) {
    if (!aligned16(yp)) return SSD_ERR_MISALIGNED;
    if (yp == y || yp == z || yp == x) return SSD_ERR_INVALID_ARG;
  }
  if (!seq_idx && (initial_states || final_states) && shape->nseqs != shape->batch) return SSD_ERR_INVALID_ARG;
  if ((initial_states || final_states) && shape->nseqs < 1) return SSD_ERR_INVALID_ARG;
  const void* ptrs[] = {x, dt, A, B, C, D, initial_states, seq_idx, y, final_states, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return SSD_ERR_MISALIGNED;
  const Layout L = make_layout(shape);
  if (workspace_bytes < L.total) return SSD_ERR_WORKSPACE_TOO_SMALL;
  ssd::Problem pb;
  fill_problem(shape, L, workspace, pb);
  if ((rc = fill_frontend(fe, pb))) return rc;
  pb.x = x; pb.dt = dt; pb.A = A; pb.Bm = B; pb.Cm = C; pb.D = D;
  pb.h0 = initial_states; pb.seq_idx = seq_idx;
  pb.y = y; pb.final = final_states; pb.z = z;
  pb.ypre = z && fe ? fe->y_pre_gate : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = is_bf16(shape);
  if (ssd::launch_prep(pb, s) != hipSuccess) return SSD_ERR_HIP;
  if (ssd::launch_state_fwd(pb, bf16, s) != hipSuccess) return SSD_ERR_HIP;
  if (final_states && ssd::launch_seqstart(pb, s) != hipSuccess) return SSD_ERR_HIP;
  if (ssd::launch_fwd_out(pb, bf16, s) != hipSuccess) return SSD_ERR_HIP;
  return SSD_OK;
}

}  // namespace

extern "C" int ssd_fwd(const ssd_shape* shape, const void* x, const float* dt, const float* A, const void* B,
                       const void* C, const float* D, const float* initial_states, const int32_t* seq_idx,
                       void* y, float* final_states, void* workspace, size_t workspace_bytes, void* stream) {
  return run_fwd(shape, nullptr, x, dt, A, B, C, D, nullptr, initial_states, seq_idx, y, final_states, workspace,
                 workspace_bytes, stream);
}

extern "C" int ssd_fwd_ex(const ssd_shape* shape, const ssd_options* fe, const void* x, const float* dt,
                          const float* A, const void* B, const void* C, const float* D, const void* z,
                          const float* initial_states, const int32_t* seq_idx, void* y, float* final_states,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return run_fwd(shape, fe, x, dt, A, B, C, D, z, initial_states, seq_idx, y, final_states, workspace,
                 workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// ssd_bwd_noalloc: ssd_bwd with its workspace in a fixed device array of
// this library (one copy per GPU, held until the process ends), for callers
// that cannot allocate.  The array's name is a host-side stand-in for a
// device symbol: its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// passed on.
// ---------------------------------------------------------------------------
namespace {

__device__ __align__(256) char scratch[SSD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device (guarded by g_scratch_mu)

int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSD_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSD_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SSD_OK;
}

}  // namespace

extern "C" int ssd_bwd_noalloc(const ssd_shape* shape, const void* x, const float* dt, const float* A,
                               const void* B, const void* C, const float* D, const void* dy,
                               const float* initial_states, const int32_t* seq_idx, void* dx, float* ddt,
                               float* dA, void* dB, void* dC, float* dD, float* d_initial_states, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (make_layout(shape).total > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws))) return rc;
  // the workspace's contents on entry do not affect the results, so nothing
  // is cleared here (the previous call's values are simply overwritten)
  return run_bwd(shape, nullptr, x, dt, A, B, C, D, nullptr, dy, initial_states, seq_idx, dx, ddt, dA, dB, dC, dD,
                 d_initial_states, nullptr, nullptr, ws, SSD_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

extern "C" int ssd_bwd_stage_count(void) { return kStages; }

extern "C" const char* ssd_bwd_stage_name(int stage) {
  return (stage >= 0 && stage < kStages) ? kStageNames[stage] : nullptr;
}
