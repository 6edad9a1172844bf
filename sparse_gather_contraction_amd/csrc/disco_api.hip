// disco_api.hip — C ABI of libdisco.so: validation, plan upload and launches.
#include <atomic>
#include <mutex>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "disco.h"
#include "kernels.hpp"
#include "plan.hpp"

namespace {

thread_local std::string g_last_error;

disco_status fail(disco_status s, const std::string &msg)
{
    g_last_error = msg;
    return s;
}

struct DevPlan {
    disco::Item *items = nullptr;
    int32_t *order = nullptr;
    disco::Seg *segs = nullptr;
    float *vals = nullptr;
    int32_t *block_ptr = nullptr;
    int32_t n_items = 0;
    int32_t L = 0, in_stride = 1;
    // the forward plan's source windows for the fp32 fused kernel (plan.hpp, FusedWindows)
    disco::FWin *fw_rows = nullptr;
    int32_t *fw_ho_ptr = nullptr, *fw_ho_len = nullptr, *fw_seg_off = nullptr;
    int32_t fw_cap = 0;  // positions per channel of the kernel's LDS area (0: no windows)
    int32_t *fw_ho_psi = nullptr;  // per latitude: its segment and value runs (null: not contiguous)
    int32_t fw_psi_bytes = 0;      // the largest latitude's psi as the kernel copies it to LDS
};

constexpr int kStagedLdsBudget = 40 * 1024;  // bytes of LDS per block (four blocks per CU)

struct DevStaged {
    bool ok = false;
    disco::Task *tasks = nullptr;
    disco::Stage *stages = nullptr;
    int32_t *stage_rows = nullptr;
    int32_t *stage_segptr = nullptr;
    disco::Seg *segs = nullptr;
    float *vals = nullptr;
    disco::Item *items = nullptr;
    int32_t n_tasks = 0;
    int32_t L = 0, row_len = 0, lrow = 0, halo = 0, rows_per_stage = 0, wpp = 4, NP = 1;
    int32_t NI = 1, G = 1, T = 3, S = 1;
};

constexpr int kTileLdsBudget = 40 * 1024;  // bytes of LDS per register-tiled workgroup (four per CU)

struct DevTile {
    bool ok = false;
    disco::Task *tasks = nullptr;
    disco::Stage *stages = nullptr;
    disco::Stage *task_first = nullptr;
    int32_t *stage_rows = nullptr;
    int32_t *stage_recptr = nullptr;
    disco::TileRec *recs = nullptr;
    disco::Item *items = nullptr;
    int32_t n_tasks = 0, n_stages = 0;
    int32_t L = 0, row_len = 0, lrow = 0, deint = 1, rows_per_stage = 0, NI = 1, G = 1, PW = 1;
    int32_t n_ws4 = 0, n_ws2 = 0, max_recs = 0;
    int32_t n_recs = 0;
};

constexpr int kLdsPerBlock = 160 * 1024;       // gfx950: a workgroup may allocate the whole 160 KiB
constexpr int kFwdMfmaStageBytes = 40 * 1024;  // two stages per forward workgroup, two workgroups per CU
constexpr int kBwdMfmaRows = 8;                // gradient rows (input row, residue) per matrix-core group

struct DevFused {
    bool ok = false;
    disco::FPiece *pieces = nullptr;
    disco::FRow *rows = nullptr;
    int32_t *descs = nullptr;
    uint16_t *adata = nullptr;    // bf16 psi
    uint16_t *adata16 = nullptr;  // fp16 psi * 2^psi16_exp (same layout)
    int32_t *ho_piece = nullptr;
    int32_t *ho_order = nullptr;
    int32_t max_piece_bytes = 0, max_resident_bytes = 0, kr = 16, psi16_exp = 0;
    uint32_t desc_bytes = 0, adata_bytes = 0;
};

template <typename T>
hipError_t upload(T **dst, const std::vector<T> &src)
{
    const size_t n = src.empty() ? 1 : src.size();
    hipError_t e = hipMalloc((void **)dst, n * sizeof(T));
    if (e != hipSuccess) return e;
    if (!src.empty()) e = hipMemcpy(*dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice);
    return e;
}

void free_plan(DevPlan &p)
{
    (void)hipFree(p.items);
    (void)hipFree(p.order);
    (void)hipFree(p.segs);
    (void)hipFree(p.vals);
    (void)hipFree(p.block_ptr);
    (void)hipFree(p.fw_rows);
    (void)hipFree(p.fw_ho_ptr);
    (void)hipFree(p.fw_ho_len);
    (void)hipFree(p.fw_seg_off);
    (void)hipFree(p.fw_ho_psi);
    p = DevPlan();
}

void free_staged(DevStaged &d)
{
    (void)hipFree(d.tasks);
    (void)hipFree(d.stages);
    (void)hipFree(d.stage_rows);
    (void)hipFree(d.stage_segptr);
    (void)hipFree(d.segs);
    (void)hipFree(d.vals);
    (void)hipFree(d.items);
    d = DevStaged();
}

hipError_t upload_staged(DevStaged &d, const disco::StagedPlan &p)
{
    d = DevStaged();
    if (!p.ok || !disco::staged_supported(p.NI, p.G, p.T, p.S)) return hipSuccess;
    hipError_t e;
    if ((e = upload(&d.tasks, p.tasks)) != hipSuccess) return e;
    if ((e = upload(&d.stages, p.stages)) != hipSuccess) return e;
    if ((e = upload(&d.stage_rows, p.stage_rows)) != hipSuccess) return e;
    if ((e = upload(&d.stage_segptr, p.stage_segptr)) != hipSuccess) return e;
    if ((e = upload(&d.segs, p.segs)) != hipSuccess) return e;
    if ((e = upload(&d.vals, p.vals)) != hipSuccess) return e;
    if ((e = upload(&d.items, p.items)) != hipSuccess) return e;
    d.ok = true;
    d.n_tasks = (int32_t)p.tasks.size();
    d.L = p.L; d.row_len = p.row_len; d.lrow = p.lrow; d.halo = p.halo; d.rows_per_stage = p.rows_per_stage;
    d.wpp = p.wpp; d.NP = p.NP; d.NI = p.NI; d.G = p.G; d.T = p.T; d.S = p.S;
    return hipSuccess;
}

void free_tile(DevTile &d)
{
    (void)hipFree(d.tasks);
    (void)hipFree(d.stages);
    (void)hipFree(d.task_first);
    (void)hipFree(d.stage_rows);
    (void)hipFree(d.stage_recptr);
    (void)hipFree(d.recs);
    (void)hipFree(d.items);
    d = DevTile();
}

hipError_t upload_tile(DevTile &d, const disco::TilePlan &p)
{
    d = DevTile();
    if (!p.ok || !disco::tile_supported(p.NI, p.G, p.PW)) return hipSuccess;
    // the kernel addresses the records through one buffer resource (32-bit byte offsets)
    if (p.recs.size() * sizeof(disco::TileRec) > (size_t)INT32_MAX) return hipSuccess;
    hipError_t e;
    if ((e = upload(&d.tasks, p.tasks)) != hipSuccess) return e;
    if ((e = upload(&d.stages, p.stages)) != hipSuccess) return e;
    if ((e = upload(&d.task_first, p.task_first)) != hipSuccess) return e;
    if ((e = upload(&d.stage_rows, p.stage_rows)) != hipSuccess) return e;
    if ((e = upload(&d.stage_recptr, p.stage_recptr)) != hipSuccess) return e;
    if ((e = upload(&d.recs, p.recs)) != hipSuccess) return e;
    if ((e = upload(&d.items, p.items)) != hipSuccess) return e;
    d.ok = true;
    d.n_tasks = (int32_t)p.tasks.size();
    d.n_stages = (int32_t)p.stages.size();
    d.L = p.L; d.row_len = p.row_len; d.lrow = p.lrow; d.deint = p.deint; d.rows_per_stage = p.rows_per_stage;
    d.NI = p.NI; d.G = p.G; d.PW = p.PW;
    d.n_ws4 = p.n_ws4; d.n_ws2 = p.n_ws2; d.max_recs = p.max_recs;
    d.n_recs = (int32_t)p.recs.size();
    return hipSuccess;
}

void free_fused(DevFused &d)
{
    (void)hipFree(d.pieces);
    (void)hipFree(d.rows);
    (void)hipFree(d.descs);
    (void)hipFree(d.adata);
    (void)hipFree(d.adata16);
    (void)hipFree(d.ho_piece);
    (void)hipFree(d.ho_order);
    d = DevFused();
}

hipError_t upload_fused(DevFused &d, const disco::FusedPlan &p)
{
    d = DevFused();
    if (!p.ok) return hipSuccess;
    hipError_t e;
    if ((e = upload(&d.pieces, p.pieces)) != hipSuccess) return e;
    if ((e = upload(&d.rows, p.rows)) != hipSuccess) return e;
    if ((e = upload(&d.descs, p.descs)) != hipSuccess) return e;
    if ((e = upload(&d.adata, p.adata)) != hipSuccess) return e;
    if ((e = upload(&d.adata16, p.adata16)) != hipSuccess) return e;
    if ((e = upload(&d.ho_piece, p.ho_piece)) != hipSuccess) return e;
    if ((e = upload(&d.ho_order, p.ho_order)) != hipSuccess) return e;
    d.ok = true;
    d.max_piece_bytes = p.max_piece_bytes;
    d.max_resident_bytes = p.max_resident_bytes;
    d.kr = p.kr;
    d.psi16_exp = p.psi16_exp;
    d.desc_bytes = (uint32_t)(p.descs.size() * sizeof(int32_t));
    d.adata_bytes = (uint32_t)(p.adata.size() * sizeof(uint16_t));
    return hipSuccess;
}

hipError_t upload_plan(DevPlan &d, const disco::GatherPlan &p)
{
    hipError_t e;
    if ((e = upload(&d.items, p.items)) != hipSuccess) return e;
    if ((e = upload(&d.order, p.order)) != hipSuccess) return e;
    if ((e = upload(&d.segs, p.segs)) != hipSuccess) return e;
    if ((e = upload(&d.vals, p.vals)) != hipSuccess) return e;
    if ((e = upload(&d.block_ptr, p.block_ptr)) != hipSuccess) return e;
    d.n_items = (int32_t)p.items.size();
    d.L = p.L;
    d.in_stride = p.in_stride;
    return hipSuccess;
}

hipError_t upload_windows(DevPlan &d, const disco::FusedWindows &w, const disco::GatherPlan &p, int K)
{
    hipError_t e;
    if (w.rows.empty()) return hipSuccess;
    for (size_t b = 0; w.psi_ok && b + 1 < p.block_ptr.size(); ++b) {  // items, segments (+ offsets), values
        const int64_t bytes = (int64_t)(p.block_ptr[b + 1] - p.block_ptr[b]) * 32 +
                              (int64_t)(w.ho_psi[4 * b + 1] - w.ho_psi[4 * b]) * 20 +
                              (int64_t)(w.ho_psi[4 * b + 3] - w.ho_psi[4 * b + 2]) * 4;
        d.fw_psi_bytes = (int32_t)std::min<int64_t>(std::max<int64_t>(d.fw_psi_bytes, bytes), INT32_MAX);
    }
    if ((e = upload(&d.fw_rows, w.rows)) != hipSuccess) return e;
    if ((e = upload(&d.fw_ho_ptr, w.ho_ptr)) != hipSuccess) return e;
    if ((e = upload(&d.fw_ho_len, w.ho_len)) != hipSuccess) return e;
    if ((e = upload(&d.fw_seg_off, w.seg_off)) != hipSuccess) return e;
    if (w.psi_ok && (e = upload(&d.fw_ho_psi, w.ho_psi)) != hipSuccess) return e;
    d.fw_cap = disco::fused_win_cap_f32(K, w.ho_len.data(), (int)w.ho_len.size());
    return hipSuccess;
}

disco_status check_device(int device)
{
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return fail(DISCO_ERR_UNSUPPORTED_DEVICE, "no HIP device is visible");
    }
    if (device < 0 || device >= n) return fail(DISCO_ERR_INVALID_ARGUMENT, "device ordinal out of range");
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
        (void)hipGetLastError();
        return fail(DISCO_ERR_HIP, "hipGetDeviceProperties failed");
    }
    const char *env = getenv("DISCO_REQUIRE_ARCH");  // test knob: the architecture prefix to accept
    const std::string want = (env && *env) ? env : "gfx950";
    const std::string arch = prop.gcnArchName;
    const bool ok = arch.compare(0, want.size(), want) == 0 && (arch.size() == want.size() || arch[want.size()] == ':');
    if (!ok) return fail(DISCO_ERR_UNSUPPORTED_DEVICE, "device architecture " + arch + " is not " + want);
    return DISCO_OK;
}

disco_status check_tensor(const disco_tensor *t, const char *name, int ndim, const int64_t *shape, int device)
{
    if (!t) return fail(DISCO_ERR_INVALID_ARGUMENT, std::string(name) + " is NULL");
    if (t->dtype != DISCO_F32 && t->dtype != DISCO_BF16 && t->dtype != DISCO_F16)
        return fail(DISCO_ERR_DTYPE, std::string(name) + " has an unsupported dtype");
    if (t->ndim != ndim) return fail(DISCO_ERR_SHAPE, std::string(name) + " has the wrong number of dimensions");
    int64_t numel = 1;
    for (int i = 0; i < ndim; ++i) {
        if (t->shape[i] != shape[i]) {
            char buf[160];
            snprintf(buf, sizeof buf, "%s dimension %d is %lld, expected %lld", name, i, (long long)t->shape[i],
                     (long long)shape[i]);
            return fail(DISCO_ERR_SHAPE, buf);
        }
        numel *= shape[i];
    }
    if (numel == 0) return DISCO_OK;
    if (!t->data) return fail(DISCO_ERR_INVALID_ARGUMENT, std::string(name) + "->data is NULL");
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, t->data) != hipSuccess) {
        (void)hipGetLastError();
        return fail(DISCO_ERR_INVALID_ARGUMENT, std::string(name) + "->data is not device memory");
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
        return fail(DISCO_ERR_INVALID_ARGUMENT, std::string(name) + "->data is not device memory");
    if (attr.device != device)
        return fail(DISCO_ERR_INVALID_ARGUMENT, std::string(name) + "->data lives on another device");
    return DISCO_OK;
}

// Byte range of a tensor view (empty when it has no elements).
void byte_range(const disco_tensor *t, uintptr_t &lo, uintptr_t &hi)
{
    int64_t n = 1;
    for (int i = 0; i < t->ndim && i < 5; ++i) n *= t->shape[i];
    const int64_t esz = t->dtype == DISCO_F32 ? 4 : 2;
    lo = (uintptr_t)t->data;
    hi = lo + (uintptr_t)(n > 0 ? n * esz : 0);
}

// DISCO_ERR_INVALID_ARGUMENT when output `o` shares bytes with `t` (both already validated).
disco_status check_disjoint(const disco_tensor *o, const char *oname, const disco_tensor *t, const char *tname)
{
    if (!o || !t || !o->data || !t->data) return DISCO_OK;
    uintptr_t a0, a1, b0, b1;
    byte_range(o, a0, a1);
    byte_range(t, b0, b1);
    if (a0 < b1 && b0 < a1)
        return fail(DISCO_ERR_INVALID_ARGUMENT, std::string(oname) + " overlaps " + tname);
    return DISCO_OK;
}

bool log_enabled()
{
    const char *e = getenv("DISCO_LOG");
    return e && *e && strcmp(e, "0") != 0;
}

}  // namespace

struct disco_psi_s {
    int device;
    int32_t K, Ho, Wo, Hi, Wi;
    int64_t nnz;
    DevPlan fwd, bwd;
    DevStaged sfwd[2], sbwd[2];  // staged plans by source dtype: [0] fp32, [1] bf16
    DevTile tfwd, tbwd;          // register-tiled fp32 plans
    DevFused fused;
    DevFused fwdm;  // phase-split plan of the matrix-core forward (bf16)
    DevFused bwdm;  // phase-split plan of the inverse CSR: the matrix-core backward (bf16)
    DevFused fused_t;  // Wi = Wo: the fused op's plan of the per-basis transpose (the fused backward's gx)
    int32_t *ho_order = nullptr;
};

namespace {

disco_status check_handle(disco_psi h)
{
    if (!h) return fail(DISCO_ERR_INVALID_ARGUMENT, "psi handle is NULL");
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) {
        (void)hipGetLastError();
        return fail(DISCO_ERR_HIP, "hipGetDevice failed");
    }
    if (cur != h->device) return fail(DISCO_ERR_INVALID_ARGUMENT, "the current device is not the psi's device");
    return DISCO_OK;
}

bool getenv_is0(const char *name)  // test knobs: "0" turns a kernel path off
{
    const char *e = getenv(name);
    return e && strcmp(e, "0") == 0;
}

// A second stream per device (default priority), created on first use and kept for the life of the
// process, for work that can overlap the caller's stream inside one call.  nullptr if it cannot be made.
hipStream_t side_stream(int device)
{
    static std::mutex mu;
    static hipStream_t streams[64] = {};
    if (device < 0 || device >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!streams[device]) {
        hipStream_t s = nullptr;
        if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        streams[device] = s;
    }
    return streams[device];
}

// A memory pool per device for short-lived temporaries of one call (stream-ordered: hipMallocFromPoolAsync
// and hipFreeAsync on the call's stream), created on first use and kept for the life of the process; it
// keeps freed memory for reuse instead of returning it at each synchronization.  nullptr if it cannot be made.
hipMemPool_t temp_pool(int device)
{
    static std::mutex mu;
    static hipMemPool_t pools[64] = {};
    if (device < 0 || device >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!pools[device]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = device;
        hipMemPool_t pool = nullptr;
        if (hipMemPoolCreate(&pool, &props) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        uint64_t keep = UINT64_MAX;
        (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        (void)hipGetLastError();
        pools[device] = pool;
    }
    return pools[device];
}

// W (Co, C, K) with K < 16 in rows of 16 (zeros past K) in a stream-ordered temporary of the device's pool,
// for the matrix-core kernels' direct W-slice loads; nullptr (and no error left pending) when K is 16,
// DISCO_PACK_W=0 (a test knob: keep the element-wise W staging) or the temporary cannot be had.  The
// caller frees a non-null result with hipFreeAsync on the same stream after its launch.
// Vector-ALU fused kernels: W in the kernel's A-operand order (launch_pack_wa_f32 for fp32 data,
// launch_pack_wa16 for 16-bit data) in a stream-ordered temporary of the device's pool, packed on `stream`;
// nullptr when nothing is needed (C or Co zero) or, with *err set, when the temporary cannot be had.  The
// caller frees a non-null result with hipFreeAsync on the same stream.
void *packed_wa(int device, const void *W, int64_t Co, int64_t C, int K, bool f32, hipStream_t stream, hipError_t *err)
{
    *err = hipSuccess;
    const int64_t n = f32 ? disco::fused_wa_f32_floats((int)Co, (int)C, K) : disco::fused_wa16_elems((int)Co, (int)C, K);
    if (n == 0) return nullptr;
    hipMemPool_t pool = temp_pool(device);
    if (!pool) {
        *err = hipErrorOutOfMemory;
        return nullptr;
    }
    void *wa = nullptr;
    if ((*err = hipMallocFromPoolAsync(&wa, (size_t)n * (f32 ? 4 : 2), pool, stream)) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    *err = f32 ? disco::launch_pack_wa_f32((const float *)W, (float *)wa, (int)Co, (int)C, K, stream)
               : disco::launch_pack_wa16(W, wa, (int)Co, (int)C, K, stream);
    return wa;
}

void *packed_w(int device, const void *W, int64_t Co, int64_t C, int K, hipStream_t stream, hipError_t *err)
{
    *err = hipSuccess;
    if (K >= 16 || Co * C == 0 || getenv_is0("DISCO_PACK_W")) return nullptr;
    hipMemPool_t pool = temp_pool(device);
    void *wp = nullptr;
    if (!pool || hipMallocFromPoolAsync(&wp, (size_t)(Co * C * 32), pool, stream) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    *err = disco::launch_pack_w16(W, wp, (int)Co, (int)C, K, stream);
    return wp;
}

bool staged_env_off()
{
    const char *e = getenv("DISCO_STAGED");  // test knob: "0" forces the plain gather kernel
    return e && strcmp(e, "0") == 0;
}

// Launch the gather over all planes, in chunks that keep the grid below 2^31 blocks.
disco_status run_gather(const DevPlan &p, const DevStaged &sp, const DevTile &tp, const void *src, void *dst,
                        int dtype, int64_t BC, int64_t src_plane, int64_t dst_plane, hipStream_t stream)
{
    if (BC == 0) return DISCO_OK;
    const size_t esz = dtype == DISCO_F32 ? 4 : 2;
    if (dtype == DISCO_F32 && tp.ok && !getenv_is0("DISCO_TILE")) {  // test knob: "0" turns the tiled gather off
        // direct loads address a plane through one buffer resource (32-bit byte offsets)
        const bool vec = ((uintptr_t)src % 16 == 0) && (src_plane % 4 == 0) && (tp.row_len % 4 == 0) &&
                         tp.L >= disco::kTileHalo && src_plane <= INT32_MAX / 4;
        // at most one workgroup per PW planes per task: keep the grid below 2^31 workgroups
        const int64_t n_pg_max = (((int64_t)1 << 31) - 1) / std::max<int32_t>(1, tp.n_tasks);
        const int64_t chunk = std::max<int64_t>(1, n_pg_max) * tp.PW;
        for (int64_t b0 = 0; b0 < BC; b0 += chunk) {
            disco::TileLaunch a;
            a.src = (const float *)src + b0 * src_plane;
            a.dst = (float *)dst + b0 * dst_plane;
            a.tasks = tp.tasks; a.stages = tp.stages; a.stage_rows = tp.stage_rows; a.stage_recptr = tp.stage_recptr;
            a.task_first = tp.task_first; a.n_stages = tp.n_stages;
            a.recs = tp.recs; a.items = tp.items;
            a.n_tasks = tp.n_tasks;
            a.BC = (int32_t)std::min<int64_t>(chunk, BC - b0);
            disco::tile_wave_split(tp.n_tasks, tp.n_recs, tp.PW, tp.n_ws4, tp.n_ws2, a.BC, a.n_ws4, a.n_ws2);
            a.max_recs = tp.max_recs; a.n_recs = tp.n_recs;
            a.src_plane = src_plane; a.dst_plane = dst_plane;
            a.L = tp.L; a.row_len = tp.row_len; a.lrow = tp.lrow; a.deint = tp.deint;
            a.rows_per_stage = tp.rows_per_stage; a.NI = tp.NI; a.G = tp.G; a.PW = tp.PW;
            a.vec = vec ? 1 : 0;
            hipError_t e = disco::launch_tile(a, stream);
            if (e != hipSuccess)
                return fail(DISCO_ERR_HIP, std::string("tiled gather launch failed: ") + hipGetErrorString(e));
        }
        return DISCO_OK;
    }
    if (sp.ok && !staged_env_off()) {
        const int align = 16 / (int)esz;
        const bool vec = ((uintptr_t)src % 16 == 0) && (src_plane % align == 0) && (sp.row_len % align == 0) &&
                         ((sp.row_len + sp.halo) % align == 0);
        const int64_t n_pg_max = (((int64_t)1 << 31) - 1) / std::max<int32_t>(1, sp.n_tasks);
        const int64_t chunk = std::max<int64_t>(1, n_pg_max) * sp.NP;
        for (int64_t b0 = 0; b0 < BC; b0 += chunk) {
            disco::StagedLaunch a;
            a.src = (const char *)src + b0 * src_plane * esz;
            a.dst = (char *)dst + b0 * dst_plane * esz;
            a.dtype = dtype;
            a.tasks = sp.tasks; a.stages = sp.stages; a.stage_rows = sp.stage_rows; a.stage_segptr = sp.stage_segptr;
            a.segs = sp.segs; a.vals = sp.vals; a.items = sp.items;
            a.n_tasks = sp.n_tasks;
            a.BC = (int32_t)std::min<int64_t>(chunk, BC - b0);
            a.src_plane = src_plane; a.dst_plane = dst_plane;
            a.L = sp.L; a.row_len = sp.row_len; a.copy_len = sp.row_len + sp.halo; a.lrow = sp.lrow;
            a.wpp = sp.wpp; a.NP = sp.NP; a.stage_elems = sp.rows_per_stage * sp.lrow; a.vec = vec ? 1 : 0;
            a.NI = sp.NI; a.G = sp.G; a.T = sp.T; a.S = sp.S;
            hipError_t e = disco::launch_staged(a, stream);
            if (e != hipSuccess)
                return fail(DISCO_ERR_HIP, std::string("staged gather launch failed: ") + hipGetErrorString(e));
        }
        return DISCO_OK;
    }
    const int64_t max_blocks = ((int64_t)1 << 31) - 1;
    const int64_t chunk = std::max<int64_t>(1, max_blocks / std::max<int32_t>(1, p.n_items));
    for (int64_t b0 = 0; b0 < BC; b0 += chunk) {
        disco::GatherLaunch a;
        a.src = (const char *)src + b0 * src_plane * esz;
        a.dst = (char *)dst + b0 * dst_plane * esz;
        a.dtype = dtype;
        a.items = p.items;
        a.order = p.order;
        a.segs = p.segs;
        a.vals = p.vals;
        a.n_items = p.n_items;
        a.BC = (int32_t)std::min<int64_t>(chunk, BC - b0);
        a.src_plane = src_plane;
        a.dst_plane = dst_plane;
        a.L = p.L;
        a.in_stride = p.in_stride;
        hipError_t e = disco::launch_gather(a, stream);
        if (e != hipSuccess) return fail(DISCO_ERR_HIP, std::string("gather launch failed: ") + hipGetErrorString(e));
    }
    return DISCO_OK;
}

// Forward contraction of B x C planes, src (B, C, Hi, Wi) -> dst (B, C, K, Ho, Wo), after validation.
// src_bs / dst_bs: elements between batches (0: the C planes of a batch follow one another).
disco_status enqueue_fwd(disco_psi h, const void *src, void *dst, int dtype, int64_t B, int64_t C, hipStream_t stream,
                         int64_t src_bs = 0, int64_t dst_bs = 0)
{
    const int d = dtype == DISCO_F32 ? 0 : 1;  // staged plan by element size
    const char *fm = getenv("DISCO_FWD_MFMA");  // test knob: "0" forces the vector-ALU gather for bf16
    if (dtype != DISCO_F32 && h->fwdm.ok && !(fm && strcmp(fm, "0") == 0)) {
        if (B * C * h->Ho == 0 || h->Wo == 0) return DISCO_OK;
        const int fch = disco::fwd_mfma_channels(h->fwdm.kr);
        if (B * h->Ho * ((C + fch - 1) / fch) * ((h->Wo + 255) / 256) >= ((int64_t)1 << 31))
            return fail(DISCO_ERR_SHAPE, "forward grid exceeds 2^31 blocks");
        disco::FwdMfmaLaunch m;
        m.x = src; m.out = dst;
        m.pieces = h->fwdm.pieces; m.rows = h->fwdm.rows; m.descs = h->fwdm.descs;
        m.f16 = dtype == DISCO_F16;
        m.adata = m.f16 ? h->fwdm.adata16 : h->fwdm.adata;
        m.scale = m.f16 ? std::ldexp(1.0f, -h->fwdm.psi16_exp) : 1.0f;
        m.ho_piece = h->fwdm.ho_piece; m.ho_order = h->fwdm.ho_order;
        m.B = (int32_t)B; m.C = (int32_t)C; m.K = h->K; m.Ho = h->Ho; m.Wo = h->Wo; m.Hi = h->Hi; m.Wi = h->Wi;
        m.s = h->Wi / h->Wo; m.kr = h->fwdm.kr; m.max_piece_bytes = h->fwdm.max_piece_bytes;
        m.desc_bytes = h->fwdm.desc_bytes; m.adata_bytes = h->fwdm.adata_bytes;
        m.om.plane = (int64_t)h->K * h->Ho * h->Wo; m.om.inverse = 0; m.om.rows = 0; m.om.wi = 0; m.om.s = 1;
        m.x_bstride = src_bs; m.out_bstride = dst_bs;
        hipError_t e = disco::launch_fwd_mfma(m, stream);
        if (e != hipSuccess) return fail(DISCO_ERR_HIP, std::string("forward launch failed: ") + hipGetErrorString(e));
        return DISCO_OK;
    }
    const int64_t sp = (int64_t)h->Hi * h->Wi, dp = (int64_t)h->K * h->Ho * h->Wo;
    if ((src_bs == 0 || src_bs == C * sp) && (dst_bs == 0 || dst_bs == C * dp))
        return run_gather(h->fwd, h->sfwd[d], h->tfwd, src, dst, dtype, B * C, sp, dp, stream);
    const size_t esz = dtype == DISCO_F32 ? 4 : 2;
    for (int64_t b = 0; b < B; ++b) {
        disco_status st = run_gather(h->fwd, h->sfwd[d], h->tfwd, (const char *)src + b * src_bs * esz,
                                     (char *)dst + b * dst_bs * esz, dtype, C, sp, dp, stream);
        if (st != DISCO_OK) return st;
    }
    return DISCO_OK;
}

// Transpose contraction of B x C planes, src (B, C, K, Ho, Wo) -> dst (B, C, Hi, Wi), after validation.
// src_bs / dst_bs: elements between batches (0: the C planes of a batch follow one another).
disco_status enqueue_bwd(disco_psi h, const void *src, void *dst, int dtype, int64_t B, int64_t C, hipStream_t stream,
                         int64_t src_bs = 0, int64_t dst_bs = 0)
{
    const int d = dtype == DISCO_F32 ? 0 : 1;  // staged plan by element size
    const char *bm = getenv("DISCO_BWD_MFMA");  // test knob: "0" forces the vector-ALU gather for bf16
    if (dtype != DISCO_F32 && h->bwdm.ok && !(bm && strcmp(bm, "0") == 0)) {
        if (B * C * h->Hi == 0 || h->Wi == 0) return DISCO_OK;
        const int fch = disco::fwd_mfma_channels(h->bwdm.kr);
        const int32_t s = h->Wi / h->Wo;
        const int32_t groups = (h->Hi * s + kBwdMfmaRows - 1) / kBwdMfmaRows;
        if (B * groups * ((C + fch - 1) / fch) * ((h->Wo + 255) / 256) >= ((int64_t)1 << 31))
            return fail(DISCO_ERR_SHAPE, "backward grid exceeds 2^31 blocks");
        disco::FwdMfmaLaunch m;
        m.x = src; m.out = dst;
        m.pieces = h->bwdm.pieces; m.rows = h->bwdm.rows; m.descs = h->bwdm.descs;
        m.f16 = dtype == DISCO_F16;
        m.adata = m.f16 ? h->bwdm.adata16 : h->bwdm.adata;
        m.scale = m.f16 ? std::ldexp(1.0f, -h->bwdm.psi16_exp) : 1.0f;
        m.ho_piece = h->bwdm.ho_piece; m.ho_order = h->bwdm.ho_order;
        m.B = (int32_t)B; m.C = (int32_t)C; m.K = kBwdMfmaRows; m.Ho = groups; m.Wo = h->Wo;
        m.Hi = h->K * h->Ho; m.Wi = h->Wo; m.s = 1; m.kr = h->bwdm.kr; m.max_piece_bytes = h->bwdm.max_piece_bytes;
        m.desc_bytes = h->bwdm.desc_bytes; m.adata_bytes = h->bwdm.adata_bytes;
        m.om.plane = (int64_t)h->Hi * h->Wi; m.om.inverse = 1; m.om.rows = h->Hi * s; m.om.wi = h->Wi; m.om.s = s;
        m.x_bstride = src_bs; m.out_bstride = dst_bs;
        hipError_t e = disco::launch_fwd_mfma(m, stream);
        if (e != hipSuccess) return fail(DISCO_ERR_HIP, std::string("backward launch failed: ") + hipGetErrorString(e));
        return DISCO_OK;
    }
    const int64_t sp = (int64_t)h->K * h->Ho * h->Wo, dp = (int64_t)h->Hi * h->Wi;
    if ((src_bs == 0 || src_bs == C * sp) && (dst_bs == 0 || dst_bs == C * dp))
        return run_gather(h->bwd, h->sbwd[d], h->tbwd, src, dst, dtype, B * C, sp, dp, stream);
    const size_t esz = dtype == DISCO_F32 ? 4 : 2;
    for (int64_t b = 0; b < B; ++b) {
        disco_status st = run_gather(h->bwd, h->sbwd[d], h->tbwd, (const char *)src + b * src_bs * esz,
                                     (char *)dst + b * dst_bs * esz, dtype, C, sp, dp, stream);
        if (st != DISCO_OK) return st;
    }
    return DISCO_OK;
}

// Workspace of the fused-convolution backward: W^T, gy^T of every batch, one channel chunk of
// g = W^T gy for every batch (and afterwards of out = F x), and the fp32 partials of dW for one
// chunk.  A chunk holds up to 1024 (c, k) rows.
struct FusedBwdLayout {
    int64_t N = 0;                 // positions Ho Wo
    int32_t Cc = 0, Mc = 0;        // channels per chunk and its rows cc K
    int32_t S = 0, kps = 0;        // position splits of dW and their length
    size_t wt = 0, gyt = 0, gbuf = 0, part = 0, total = 0;  // byte offsets and total
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// `cap`: the largest workspace the caller can give; channel chunks shrink (down to one channel) until
// the layout fits, if it can.
// The fused backward's gx takes one fused launch over the per-basis transpose of psi (Wi = Wo, plan built);
// otherwise W^T gy per channel chunk and the transpose contraction.
bool bwd_gx_fused(const disco_psi_s *h)
{
    return h->fused_t.ok && h->Wi == h->Wo && !getenv_is0("DISCO_BWD_FUSED");  // test knob: "0" keeps W^T gy
}

FusedBwdLayout fused_bwd_layout(const disco_psi_s *h, int64_t B, int64_t C, int64_t Co, size_t cap = SIZE_MAX)
{
    const int64_t K = h->K;
    const bool gx_fused = bwd_gx_fused(h);
    const int64_t N = (int64_t)h->Ho * h->Wo;
    // up to 1024 (c, k) rows per chunk (1024 measured 6 % faster than 512 at 721x1440: fewer launches,
    // gy^T read fewer times), and few enough that one batch's chunk stays below 2 GiB
    const int64_t rows = std::min<int64_t>(1024, (((int64_t)1 << 31) - 1) / std::max<int64_t>(2 * N, 1));
    int64_t cc = std::max<int64_t>(1, std::min<int64_t>(std::max<int64_t>(C, 1), rows / std::max<int64_t>(K, 1)));
    for (;;) {
        FusedBwdLayout L;
        L.N = N;
        L.Cc = (int32_t)cc;
        L.Mc = (int32_t)(L.Cc * K);
        // at most 64 splits: fewer fp32 partials to sum (64 measured 2 % faster than 256 per backward
        // at 721x1440 and still >= one workgroup per CU there)
        const int64_t per = std::max<int64_t>(1, (L.N + 63) / 64);
        L.kps = (int32_t)((per + 31) / 32 * 32);
        L.S = (int32_t)std::max<int64_t>(1, (L.N + L.kps - 1) / L.kps);
        size_t off = 0;
        // W^T (C K, Co), or W' (C, Co, 16) for the fused gx; gy^T only for the W^T gy products
        L.wt = off;   off = align256(off + (size_t)C * (gx_fused ? 16 : K) * Co * 2);
        L.gyt = off;  off = align256(off + (gx_fused ? 0 : (size_t)B * L.N * Co * 2));
        L.gbuf = off; off = align256(off + (size_t)B * L.Mc * L.N * 2);
        L.part = off; off = align256(off + (size_t)B * L.S * Co * L.Mc * 4);
        L.total = off;
        if (L.total <= cap || cc == 1) return L;
        cc = (cc + 1) / 2;
    }
}

// File-scope scratch of disco_fused_conv_bwd_noalloc: each device that runs the library holds its own
// copy until the process ends.  In host code `scratch` only names the symbol; its device address is
// looked up once per device (init_scratch, called by disco_psi_create with the device current) and
// that pointer is what the kernels receive.
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {};

// The current device must be `device`.
disco_status init_scratch(int device)
{
    if (device < 0 || device >= 64) return fail(DISCO_ERR_INVALID_ARGUMENT, "device ordinal out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[device]) return DISCO_OK;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
        (void)hipGetLastError();
        return fail(DISCO_ERR_HIP, std::string("cannot look up the scratch array: ") + hipGetErrorString(e));
    }
    g_scratch_ptr[device] = p;
    return DISCO_OK;
}

void *scratch_ptr(int device)
{
    if (device < 0 || device >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_ptr[device];
}

}  // namespace

extern "C" {

const char *disco_last_error(void) { return g_last_error.c_str(); }

disco_status disco_psi_create(const disco_csr_desc *csr, int device, disco_psi *out_handle)
{
    if (!csr || !out_handle) return fail(DISCO_ERR_INVALID_ARGUMENT, "csr or out_handle is NULL");
    *out_handle = nullptr;
    disco::CSRView v{csr->K, csr->Ho, csr->Wo, csr->Hi, csr->Wi, csr->nnz, csr->row_ptr, csr->col_hi, csr->col_wi, csr->val};
    int code = 0;
    std::string msg = disco::validate_csr(v, &code);
    if (code != 0) return fail((disco_status)code, msg);
    disco_status st = check_device(device);
    if (st != DISCO_OK) return st;

    disco::GatherPlan fp, bp;
    disco::FusedWindows fw;
    try {
        disco::build_forward_plan(v, fp);
        disco::build_backward_plan(v, bp);
        disco::build_fused_windows(fp, disco::fused_tile_px(), fw);
    } catch (const std::bad_alloc &) {
        return fail(DISCO_ERR_OOM, "host allocation failed while building the plan");
    }
    disco::StagedPlan sfp[2], sbp[2];
    try {
        for (int d = 0; d < 2; ++d) {
            const int esz = d ? 2 : 4;
            disco::build_staged_plan(v, fp, false, esz, kStagedLdsBudget, sfp[d]);
            disco::build_staged_plan(v, bp, true, esz, kStagedLdsBudget, sbp[d]);
        }
    } catch (const std::bad_alloc &) {
        return fail(DISCO_ERR_OOM, "host allocation failed while building the staged plan");
    }
    disco::TilePlan tfp, tbp;
    try {
        int tile_lds = kTileLdsBudget;
        const char *tl = getenv("DISCO_TILE_LDS");  // tuning knob: LDS bytes per tiled workgroup
        if (tl && atoi(tl) >= 4096 && atoi(tl) <= 64 * 1024) tile_lds = atoi(tl);
        disco::build_tile_plan(v, fp, false, tile_lds, tfp);
        disco::build_tile_plan(v, bp, true, tile_lds, tbp);
    } catch (const std::bad_alloc &) {
        return fail(DISCO_ERR_OOM, "host allocation failed while building the tiled plan");
    }
    disco::FusedPlan fup, fwp, bwp, fut;
    try {
        // two piece stage buffers share what the W slice leaves of the workgroup's LDS
        const int ch = disco::fused_mfma_channels_per_chunk();
        const int budget = ((kLdsPerBlock - (int)disco::fused_mfma_reserved_bytes()) / 2) & ~15;
        disco::PhasePlanParams prm;
        prm.kr = 16;
        prm.ch = ch;
        prm.piece_budget = budget;
        prm.xch_bytes = disco::fused_mfma_exchange_bytes();
        const char *pcp = getenv("DISCO_PSI_COPIES");  // tuning knob: psi copies for odd strides (1, 2 or 3)
        if (pcp && (pcp[0] == '1' || pcp[0] == '2' || pcp[0] == '3') && pcp[1] == 0) prm.psi_copies = pcp[0] - '0';
        disco::build_phase_plan(v, prm, fup);
        if (fup.ok && csr->Wi == csr->Wo) {
            // the fused backward's gx = the fused op over the per-basis transpose of psi (same grid both ways)
            disco::TransposedCSR tr;
            disco::build_transposed_csr(v, tr);
            disco::build_phase_plan(tr.view, prm, fut);
        }
        disco::PhasePlanParams fprm;
        fprm.kr = csr->K <= 8 ? 8 : 16;
        fprm.ch = disco::fwd_mfma_channels(fprm.kr);
        fprm.piece_budget = kFwdMfmaStageBytes;
        fprm.xch_bytes = 0;
        fprm.allow_resident = false;
        disco::build_phase_plan(v, fprm, fwp);
        disco::InverseCSR inv;
        disco::build_inverse_csr(v, kBwdMfmaRows, inv);
        disco::PhasePlanParams bprm = fprm;
        bprm.kr = kBwdMfmaRows;
        bprm.ch = disco::fwd_mfma_channels(bprm.kr);
        bprm.psi_copies = prm.psi_copies;
        disco::build_phase_plan(inv.view, bprm, bwp);
    } catch (const std::bad_alloc &) {
        return fail(DISCO_ERR_OOM, "host allocation failed while building the fused plan");
    }
    // latitudes ordered by forward work, heaviest first (fused launch order)
    std::vector<int64_t> work(csr->Ho, 0);
    for (int32_t ho = 0; ho < csr->Ho; ++ho)
        for (int32_t i = fp.block_ptr[ho]; i < fp.block_ptr[ho + 1]; ++i)
            for (int32_t s = fp.items[i].seg_begin; s < fp.items[i].seg_end; ++s) work[ho] += (int64_t)fp.segs[s].m * fp.items[i].G;
    std::vector<int32_t> ho_order(csr->Ho);
    for (int32_t i = 0; i < csr->Ho; ++i) ho_order[i] = i;
    std::stable_sort(ho_order.begin(), ho_order.end(), [&](int32_t a, int32_t b) { return work[a] > work[b]; });

    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess || hipSetDevice(device) != hipSuccess) {
        (void)hipGetLastError();
        return fail(DISCO_ERR_HIP, "cannot select the device");
    }
    if ((st = init_scratch(device)) != DISCO_OK) {
        (void)hipSetDevice(prev);
        return st;
    }
    disco_psi h = new (std::nothrow) disco_psi_s();
    if (!h) {
        (void)hipSetDevice(prev);
        return fail(DISCO_ERR_OOM, "host allocation failed");
    }
    h->device = device;
    h->K = csr->K; h->Ho = csr->Ho; h->Wo = csr->Wo; h->Hi = csr->Hi; h->Wi = csr->Wi;
    h->nnz = csr->nnz;
    hipError_t e = upload_plan(h->fwd, fp);
    if (e == hipSuccess) e = upload_windows(h->fwd, fw, fp, csr->K);
    if (e == hipSuccess) e = upload_plan(h->bwd, bp);
    if (e == hipSuccess) e = upload(&h->ho_order, ho_order);
    for (int d = 0; d < 2 && e == hipSuccess; ++d) {
        e = upload_staged(h->sfwd[d], sfp[d]);
        if (e == hipSuccess) e = upload_staged(h->sbwd[d], sbp[d]);
    }
    if (e == hipSuccess) e = upload_tile(h->tfwd, tfp);
    if (e == hipSuccess) e = upload_tile(h->tbwd, tbp);
    if (e == hipSuccess) e = upload_fused(h->fused, fup);
    if (e == hipSuccess) e = upload_fused(h->fwdm, fwp);
    if (e == hipSuccess) e = upload_fused(h->bwdm, bwp);
    if (e == hipSuccess) e = upload_fused(h->fused_t, fut);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        free_plan(h->fwd);
        free_plan(h->bwd);
        free_fused(h->fused);
        free_fused(h->fwdm);
        free_fused(h->bwdm);
        free_fused(h->fused_t);
        free_tile(h->tfwd);
        free_tile(h->tbwd);
        for (int d = 0; d < 2; ++d) {
            free_staged(h->sfwd[d]);
            free_staged(h->sbwd[d]);
        }
        (void)hipFree(h->ho_order);
        delete h;
        (void)hipSetDevice(prev);
        return fail(e == hipErrorOutOfMemory ? DISCO_ERR_OOM : DISCO_ERR_HIP,
                    std::string("plan upload failed: ") + hipGetErrorString(e));
    }
    (void)hipSetDevice(prev);
    if (log_enabled())
        fprintf(stderr,
                "[disco] psi K=%d Ho=%d Wo=%d Hi=%d Wi=%d nnz=%lld | fwd: %zu items %zu segs %zu vals | "
                "bwd: %zu items %zu segs | staged bf16 fwd %s (%zu tasks, %zu stages, T=%d G=%d) bwd %s (%zu tasks, "
                "%zu stages)\n",
                h->K, h->Ho, h->Wo, h->Hi, h->Wi, (long long)h->nnz, fp.items.size(), fp.segs.size(), fp.vals.size(),
                bp.items.size(), bp.segs.size(), h->sfwd[1].ok ? "on" : "off", sfp[1].tasks.size(),
                sfp[1].stages.size(), sfp[1].T, sfp[1].G, h->sbwd[1].ok ? "on" : "off", sbp[1].tasks.size(),
                sbp[1].stages.size());
    if (log_enabled())
        fprintf(stderr, "[disco] fused packed plan %s: %zu pieces, %lld blocks, largest stage %d bytes, window %d\n",
                fup.ok ? "on" : "off", fup.pieces.size(), (long long)fup.mfma_blocks, fup.max_piece_bytes, fup.max_win);
    *out_handle = h;
    return DISCO_OK;
}

disco_status disco_psi_destroy(disco_psi h)
{
    if (!h) return DISCO_OK;
    int prev = -1;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(h->device);
    free_plan(h->fwd);
    free_plan(h->bwd);
    for (int d = 0; d < 2; ++d) {
        free_staged(h->sfwd[d]);
        free_staged(h->sbwd[d]);
    }
    free_fused(h->fused);
    free_fused(h->fwdm);
    free_fused(h->bwdm);
    free_fused(h->fused_t);
    free_tile(h->tfwd);
    free_tile(h->tbwd);
    (void)hipFree(h->ho_order);
    (void)hipSetDevice(prev);
    delete h;
    return DISCO_OK;
}

disco_status disco_fwd(disco_psi h, const disco_tensor *x, disco_tensor *out, void *stream)
{
    disco_status st = check_handle(h);
    if (st != DISCO_OK) return st;
    if (!x || !out) return fail(DISCO_ERR_INVALID_ARGUMENT, "x or out is NULL");
    if (x->ndim != 4) return fail(DISCO_ERR_SHAPE, "x must be (B, C, Hi, Wi)");
    const int64_t B = x->shape[0], C = x->shape[1];
    if (B < 0 || C < 0) return fail(DISCO_ERR_SHAPE, "negative batch or channel count");
    const int64_t xs[4] = {B, C, h->Hi, h->Wi};
    const int64_t os[5] = {B, C, h->K, h->Ho, h->Wo};
    if ((st = check_tensor(x, "x", 4, xs, h->device)) != DISCO_OK) return st;
    if ((st = check_tensor(out, "out", 5, os, h->device)) != DISCO_OK) return st;
    if (x->dtype != out->dtype) return fail(DISCO_ERR_DTYPE, "x and out dtypes differ");
    if ((st = check_disjoint(out, "out", x, "x")) != DISCO_OK) return st;
    return enqueue_fwd(h, x->data, out->data, x->dtype, B, C, (hipStream_t)stream);
}

disco_status disco_bwd(disco_psi h, const disco_tensor *gout, disco_tensor *gx, void *stream)
{
    disco_status st = check_handle(h);
    if (st != DISCO_OK) return st;
    if (!gout || !gx) return fail(DISCO_ERR_INVALID_ARGUMENT, "gout or gx is NULL");
    if (gout->ndim != 5) return fail(DISCO_ERR_SHAPE, "gout must be (B, C, K, Ho, Wo)");
    const int64_t B = gout->shape[0], C = gout->shape[1];
    if (B < 0 || C < 0) return fail(DISCO_ERR_SHAPE, "negative batch or channel count");
    const int64_t gs[5] = {B, C, h->K, h->Ho, h->Wo};
    const int64_t xs[4] = {B, C, h->Hi, h->Wi};
    if ((st = check_tensor(gout, "gout", 5, gs, h->device)) != DISCO_OK) return st;
    if ((st = check_tensor(gx, "gx", 4, xs, h->device)) != DISCO_OK) return st;
    if (gout->dtype != gx->dtype) return fail(DISCO_ERR_DTYPE, "gout and gx dtypes differ");
    if ((st = check_disjoint(gx, "gx", gout, "gout")) != DISCO_OK) return st;
    return enqueue_bwd(h, gout->data, gx->data, gout->dtype, B, C, (hipStream_t)stream);
}

namespace {

// The fused convolution; with `save` it also writes the contraction (B, C, K, Ho, Wo).
disco_status fused_conv_impl(disco_psi h, const disco_tensor *x, const disco_tensor *W, disco_tensor *y,
                             disco_tensor *save, void *stream)
{
    disco_status st = check_handle(h);
    if (st != DISCO_OK) return st;
    if (!x || !W || !y) return fail(DISCO_ERR_INVALID_ARGUMENT, "x, W or y is NULL");
    if (x->ndim != 4) return fail(DISCO_ERR_SHAPE, "x must be (B, C, Hi, Wi)");
    if (W->ndim != 3) return fail(DISCO_ERR_SHAPE, "W must be (Co, C, K)");
    const int64_t B = x->shape[0], C = x->shape[1], Co = W->shape[0];
    if (B < 0 || C < 0 || Co < 0) return fail(DISCO_ERR_SHAPE, "negative batch or channel count");
    if (h->K > disco::fused_max_k()) return fail(DISCO_ERR_SHAPE, "the fused kernel supports K <= 64");
    const int64_t xs[4] = {B, C, h->Hi, h->Wi};
    const int64_t ws[3] = {Co, C, h->K};
    const int64_t ys[4] = {B, Co, h->Ho, h->Wo};
    if ((st = check_tensor(x, "x", 4, xs, h->device)) != DISCO_OK) return st;
    if ((st = check_tensor(W, "W", 3, ws, h->device)) != DISCO_OK) return st;
    if ((st = check_tensor(y, "y", 4, ys, h->device)) != DISCO_OK) return st;
    if (x->dtype != W->dtype || x->dtype != y->dtype) return fail(DISCO_ERR_DTYPE, "x, W and y dtypes differ");
    if (save) {
        const int64_t os[5] = {B, C, h->K, h->Ho, h->Wo};
        if ((st = check_tensor(save, "out", 5, os, h->device)) != DISCO_OK) return st;
        if (save->dtype != x->dtype) return fail(DISCO_ERR_DTYPE, "x and out dtypes differ");
        if ((st = check_disjoint(save, "out", x, "x")) != DISCO_OK) return st;
        if ((st = check_disjoint(save, "out", W, "W")) != DISCO_OK) return st;
        if ((st = check_disjoint(save, "out", y, "y")) != DISCO_OK) return st;
    }
    if ((st = check_disjoint(y, "y", x, "x")) != DISCO_OK) return st;
    if ((st = check_disjoint(y, "y", W, "W")) != DISCO_OK) return st;
    // every check before anything is enqueued (the fallback below writes `out` first)
    if (B * h->Ho * ((Co + 255) / 256) * ((h->Wo + 63) / 64) >= ((int64_t)1 << 31))
        return fail(DISCO_ERR_SHAPE, "fused grid exceeds 2^31 blocks");
    // the vector-ALU fused kernels (fp32 data, or shapes outside the matrix-core plan) take W packed for
    // their einsum: packed before anything else is enqueued
    const bool valu = x->dtype == DISCO_F32 || !h->fused.ok || getenv_is0("DISCO_FUSED_MFMA");
    void *wa = nullptr;
    if (valu && B * Co * h->Ho > 0 && h->Wo > 0) {
        hipError_t e = hipSuccess;
        wa = packed_wa(h->device, W->data, Co, C, h->K, x->dtype == DISCO_F32, (hipStream_t)stream, &e);
        if (e != hipSuccess) {
            if (wa) (void)hipFreeAsync(wa, (hipStream_t)stream);
            return fail(e == hipErrorOutOfMemory ? DISCO_ERR_OOM : DISCO_ERR_HIP,
                        std::string("fused op: packing W failed: ") + hipGetErrorString(e));
        }
    }
    if (save && B * C * h->Ho * h->Wo > 0 && (B * Co == 0 || valu)) {
        // no matrix-core fused kernel to keep the contraction from: the forward writes it
        if ((st = enqueue_fwd(h, x->data, save->data, x->dtype, B, C, (hipStream_t)stream)) != DISCO_OK) {
            if (wa) (void)hipFreeAsync(wa, (hipStream_t)stream);
            return st;
        }
    }
    if (B * Co * h->Ho == 0 || h->Wo == 0) return DISCO_OK;
    if (!valu) {  // DISCO_FUSED_MFMA=0 (test knob) forces the VALU-contraction fused kernel
        disco::FusedMfmaLaunch m;
        m.x = x->data; m.W = W->data; m.y = y->data;
        m.pieces = h->fused.pieces; m.rows = h->fused.rows; m.descs = h->fused.descs;
        m.f16 = x->dtype == DISCO_F16;
        m.adata = m.f16 ? h->fused.adata16 : h->fused.adata;
        m.scale = m.f16 ? std::ldexp(1.0f, -h->fused.psi16_exp) : 1.0f;
        m.ho_piece = h->fused.ho_piece; m.ho_order = h->fused.ho_order;
        m.B = (int32_t)B; m.C = (int32_t)C; m.Co = (int32_t)Co; m.K = h->K;
        m.Ho = h->Ho; m.Wo = h->Wo; m.Hi = h->Hi; m.Wi = h->Wi; m.s = h->Wi / h->Wo;
        m.max_piece_bytes = h->fused.max_piece_bytes;
        m.max_resident_bytes = h->fused.max_resident_bytes;
        m.desc_bytes = h->fused.desc_bytes; m.adata_bytes = h->fused.adata_bytes;
        m.save = save ? save->data : nullptr;
        // K < 16: W's rows of K elements cannot be loaded as 16-byte runs, so a stream-ordered temporary
        // holds W in rows of 16 (zeros past K) for the kernel's direct W-slice loads; without the
        // temporary the kernel stages W element by element (same values, same result)
        hipStream_t sm = (hipStream_t)stream;
        hipError_t e = hipSuccess;
        void *wp = packed_w(h->device, W->data, Co, C, h->K, sm, &e);
        if (wp && e == hipSuccess) {
            m.W = wp;
            m.w16 = true;
        }
        if (e == hipSuccess) e = disco::launch_fused_mfma(m, sm);
        if (wp) {
            const hipError_t ef = hipFreeAsync(wp, sm);
            if (e == hipSuccess) e = ef;
        }
        if (e != hipSuccess)
            return fail(DISCO_ERR_HIP, std::string("fused launch failed: ") + hipGetErrorString(e));
        return DISCO_OK;
    }
    disco::FusedLaunch a;
    a.x = x->data;
    a.W = W->data;
    a.y = y->data;
    a.f16 = x->dtype == DISCO_F16;
    a.f32 = x->dtype == DISCO_F32;
    a.items = h->fwd.items;
    a.block_ptr = h->fwd.block_ptr;
    a.ho_order = h->ho_order;
    a.segs = h->fwd.segs;
    a.vals = h->fwd.vals;
    a.B = (int32_t)B; a.C = (int32_t)C; a.Co = (int32_t)Co; a.K = h->K;
    a.Ho = h->Ho; a.Wo = h->Wo; a.Hi = h->Hi; a.Wi = h->Wi;
    a.in_stride = h->fwd.in_stride;
    if (x->dtype == DISCO_F32) a.Wa = (const float *)wa;
    else a.Wa16 = wa;
    if (!getenv_is0("DISCO_FUSED_WIN")) {  // test knob: "0" makes the vector-ALU fused kernels read x from memory
        a.fw_rows = h->fwd.fw_rows;
        a.fw_ho_ptr = h->fwd.fw_ho_ptr;
        a.fw_ho_len = h->fwd.fw_ho_len;
        a.fw_seg_off = h->fwd.fw_seg_off;
        a.fw_cap = h->fwd.fw_cap;
        if (!getenv_is0("DISCO_FUSED_PSI_LDS")) {  // test knob: "0" reads psi from memory
            a.fw_ho_psi = h->fwd.fw_ho_psi;
            a.fw_psi_bytes = h->fwd.fw_psi_bytes;
        }
    }
    hipError_t e = disco::launch_fused(a, (hipStream_t)stream);
    if (wa) {
        const hipError_t ef = hipFreeAsync(wa, (hipStream_t)stream);
        if (e == hipSuccess) e = ef;
    }
    if (e != hipSuccess) return fail(DISCO_ERR_HIP, std::string("fused launch failed: ") + hipGetErrorString(e));
    return DISCO_OK;
}

}  // namespace

disco_status disco_fused_conv(disco_psi h, const disco_tensor *x, const disco_tensor *W, disco_tensor *y,
                              void *stream)
{
    return fused_conv_impl(h, x, W, y, nullptr, stream);
}

disco_status disco_fused_conv_save(disco_psi h, const disco_tensor *x, const disco_tensor *W, disco_tensor *y,
                                   disco_tensor *out, void *stream)
{
    if (!out) return fail(DISCO_ERR_INVALID_ARGUMENT, "out is NULL");
    return fused_conv_impl(h, x, W, y, out, stream);
}


disco_status disco_einsum(const disco_tensor *W, const disco_tensor *t, disco_tensor *y, void *stream)
{
    if (!W || !t || !y) return fail(DISCO_ERR_INVALID_ARGUMENT, "W, t or y is NULL");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(DISCO_ERR_HIP, "hipGetDevice failed");
    }
    // the architecture check of a device runs once per process (its answer cannot change)
    static std::atomic<int> arch_ok[64];
    if (dev < 0 || dev >= 64) return fail(DISCO_ERR_INVALID_ARGUMENT, "device ordinal out of range");
    if (arch_ok[dev].load() != 1) {
        disco_status st = check_device(dev);
        if (st != DISCO_OK) return st;
        arch_ok[dev].store(1);
    }
    if (t->ndim != 5) return fail(DISCO_ERR_SHAPE, "t must be (B, C, K, Ho, Wo)");
    if (W->ndim != 3) return fail(DISCO_ERR_SHAPE, "W must be (Co, C, K)");
    const int64_t B = t->shape[0], C = t->shape[1], K = t->shape[2], Ho = t->shape[3], Wo = t->shape[4];
    const int64_t Co = W->shape[0];
    if (B < 0 || C < 0 || K < 0 || Ho < 0 || Wo < 0 || Co < 0) return fail(DISCO_ERR_SHAPE, "negative dimension");
    if (K > 16) return fail(DISCO_ERR_SHAPE, "the einsum kernel supports K <= 16");
    if (B > INT32_MAX || C > INT32_MAX || Co > INT32_MAX) return fail(DISCO_ERR_SHAPE, "dimension exceeds 2^31");
    const int64_t ts[5] = {B, C, K, Ho, Wo};
    const int64_t ws[3] = {Co, C, K};
    const int64_t ys[4] = {B, Co, Ho, Wo};
    disco_status st;
    if ((st = check_tensor(t, "t", 5, ts, dev)) != DISCO_OK) return st;
    if ((st = check_tensor(W, "W", 3, ws, dev)) != DISCO_OK) return st;
    if ((st = check_tensor(y, "y", 4, ys, dev)) != DISCO_OK) return st;
    if (t->dtype != W->dtype || t->dtype != y->dtype) return fail(DISCO_ERR_DTYPE, "t, W and y dtypes differ");
    if ((st = check_disjoint(y, "y", t, "t")) != DISCO_OK) return st;
    if ((st = check_disjoint(y, "y", W, "W")) != DISCO_OK) return st;
    if (t->dtype == DISCO_F32) return fail(DISCO_ERR_DTYPE, "the einsum supports bf16 and fp16 only");
    const int64_t HW = Ho * Wo;
    if (B * Co * HW == 0) return DISCO_OK;
    if (B * ((Co + 255) / 256) * ((HW + 255) / 256) >= ((int64_t)1 << 31))
        return fail(DISCO_ERR_SHAPE, "einsum grid exceeds 2^31 blocks");
    disco::EinsumLaunch a;
    a.t = t->data; a.W = W->data; a.y = y->data;
    a.B = (int32_t)B; a.C = (int32_t)C; a.Co = (int32_t)Co; a.K = (int32_t)K;
    a.HW = HW;
    a.f16 = t->dtype == DISCO_F16;
    hipStream_t sm = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    void *wp = packed_w(dev, W->data, Co, C, (int)K, sm, &e);  // K < 16: W in rows of 16 (see packed_w)
    if (wp && e == hipSuccess) {
        a.W = wp;
        a.w16 = true;
    }
    if (e == hipSuccess) e = disco::launch_einsum_mfma(a, sm);
    if (wp) {
        const hipError_t ef = hipFreeAsync(wp, sm);
        if (e == hipSuccess) e = ef;
    }
    if (e != hipSuccess) return fail(DISCO_ERR_HIP, std::string("einsum launch failed: ") + hipGetErrorString(e));
    return DISCO_OK;
}

disco_status disco_fused_conv_bwd_workspace(disco_psi h, int64_t B, int64_t C, int64_t Co, size_t *bytes)
{
    disco_status st = check_handle(h);
    if (st != DISCO_OK) return st;
    if (!bytes) return fail(DISCO_ERR_INVALID_ARGUMENT, "bytes is NULL");
    if (B < 0 || C < 0 || Co < 0) return fail(DISCO_ERR_SHAPE, "negative batch or channel count");
    *bytes = fused_bwd_layout(h, B, C, Co).total;
    return DISCO_OK;
}

namespace {

// Backward of the fused convolution; the dW operand out = F x is recomputed from x, or taken from
// `saved` (the contraction disco_fused_conv_save wrote) when x is NULL.
// `cap` < SIZE_MAX: the workspace is the library's scratch array of `cap` bytes (the no-allocation
// variant): the layout shrinks its channel chunks to fit, and a shape that cannot fit is refused.
disco_status fused_conv_bwd_impl(disco_psi h, const disco_tensor *x, const disco_tensor *saved, const disco_tensor *W,
                                 const disco_tensor *gy, disco_tensor *gx, disco_tensor *dW, void *workspace,
                                 size_t workspace_bytes, void *stream, size_t cap = SIZE_MAX)
{
    disco_status st = check_handle(h);
    if (st != DISCO_OK) return st;
    const disco_tensor *src = x ? x : saved;
    if (!src || !W || !gy || !gx || !dW)
        return fail(DISCO_ERR_INVALID_ARGUMENT, x || !saved ? "x, W, gy, gx or dW is NULL" : "out, W, gy, gx or dW is NULL");
    if (x && x->ndim != 4) return fail(DISCO_ERR_SHAPE, "x must be (B, C, Hi, Wi)");
    if (!x && saved->ndim != 5) return fail(DISCO_ERR_SHAPE, "out must be (B, C, K, Ho, Wo)");
    if (W->ndim != 3) return fail(DISCO_ERR_SHAPE, "W must be (Co, C, K)");
    const int64_t B = src->shape[0], C = src->shape[1], Co = W->shape[0];
    if (B < 0 || C < 0 || Co < 0) return fail(DISCO_ERR_SHAPE, "negative batch or channel count");
    const int64_t xs[4] = {B, C, h->Hi, h->Wi};
    const int64_t os[5] = {B, C, h->K, h->Ho, h->Wo};
    const int64_t ws[3] = {Co, C, h->K};
    const int64_t ys[4] = {B, Co, h->Ho, h->Wo};
    if (x && (st = check_tensor(x, "x", 4, xs, h->device)) != DISCO_OK) return st;
    if (!x && (st = check_tensor(saved, "out", 5, os, h->device)) != DISCO_OK) return st;
    if ((st = check_tensor(W, "W", 3, ws, h->device)) != DISCO_OK) return st;
    if ((st = check_tensor(gy, "gy", 4, ys, h->device)) != DISCO_OK) return st;
    if ((st = check_tensor(gx, "gx", 4, xs, h->device)) != DISCO_OK) return st;
    if ((st = check_tensor(dW, "dW", 3, ws, h->device)) != DISCO_OK) return st;
    if (src->dtype != W->dtype || src->dtype != gy->dtype || src->dtype != gx->dtype || src->dtype != dW->dtype)
        return fail(DISCO_ERR_DTYPE, x ? "x, W, gy, gx and dW dtypes differ" : "out, W, gy, gx and dW dtypes differ");
    if (src->dtype != DISCO_BF16 && src->dtype != DISCO_F16)
        return fail(DISCO_ERR_DTYPE, "the fused convolution backward supports bf16 and fp16 only");
    const int dt = src->dtype;
    const bool f16 = dt == DISCO_F16;
    {
        const disco_tensor *ins[3] = {src, W, gy};
        const char *names[3] = {x ? "x" : "out", "W", "gy"};
        for (int i = 0; i < 3; ++i) {
            if ((st = check_disjoint(gx, "gx", ins[i], names[i])) != DISCO_OK) return st;
            if ((st = check_disjoint(dW, "dW", ins[i], names[i])) != DISCO_OK) return st;
        }
        if ((st = check_disjoint(dW, "dW", gx, "gx")) != DISCO_OK) return st;
    }
    if (h->K > 256) return fail(DISCO_ERR_SHAPE, "the fused convolution backward supports K <= 256");
    const FusedBwdLayout L = fused_bwd_layout(h, B, C, Co, cap);
    if (Co % 8 != 0 || L.N % 8 != 0)
        return fail(DISCO_ERR_SHAPE, "the fused convolution backward needs Co and Ho*Wo to be multiples of 8");
    const int64_t lim = (int64_t)1 << 31;
    if (L.N * Co * 2 >= lim || (int64_t)L.Mc * L.N * 2 >= lim || C * h->K * Co * 2 >= lim)
        return fail(DISCO_ERR_SHAPE, "a per-batch operand of the fused convolution backward exceeds 2 GiB");
    if (cap != SIZE_MAX && L.total > cap) {
        char buf[200];
        snprintf(buf, sizeof buf,
                 "this backward needs %zu bytes of scratch; the no-allocation entry point holds at most %zu",
                 L.total, cap);
        return fail(DISCO_ERR_SHAPE, buf);
    }
    if (!workspace && L.total > 0) return fail(DISCO_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if (workspace_bytes < L.total)
        return fail(DISCO_ERR_INVALID_ARGUMENT, "workspace is smaller than disco_fused_conv_bwd_workspace reports");
    if ((uintptr_t)workspace % 256 != 0) return fail(DISCO_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    hipStream_t sm = (hipStream_t)stream;
    auto hipfail = [&](hipError_t e, const char *what) {
        return fail(DISCO_ERR_HIP, std::string(what) + " launch failed: " + hipGetErrorString(e));
    };
    char *ws_c = (char *)workspace;
    uint16_t *wt = (uint16_t *)(ws_c + L.wt), *gyt = (uint16_t *)(ws_c + L.gyt), *gbuf = (uint16_t *)(ws_c + L.gbuf);
    float *part = (float *)(ws_c + L.part);
    const uint16_t *xp = x ? (const uint16_t *)x->data : nullptr, *gyp = (const uint16_t *)gy->data;
    const uint16_t *svp = x ? nullptr : (const uint16_t *)saved->data;  // saved contraction (B, C, K, N)
    uint16_t *gxp = (uint16_t *)gx->data;
    const int64_t K = h->K, N = L.N, CK = C * K, plane_in = (int64_t)h->Hi * h->Wi;
    hipError_t e;
    // gx: with Wi = Wo the fused op over the per-basis transpose of psi, with W'[c, o, k] = W[o, c, k]
    // (gx[c] = sum_{o,k} W[o,c,k] F_k^T gy[o]); otherwise W^T gy per channel chunk, then the transpose
    // contraction of that chunk
    const bool gx_fused = bwd_gx_fused(h);
    if (gx_fused && B * h->Hi * ((C + 255) / 256) * ((h->Wo + 63) / 64) >= ((int64_t)1 << 31))
        return fail(DISCO_ERR_SHAPE, "fused backward grid exceeds 2^31 blocks");
    if (gx_fused) {
        if ((e = disco::launch_permute_w16(W->data, wt, (int)Co, (int)C, (int)K, sm)) != hipSuccess)
            return hipfail(e, "W permutation");
    } else {
        // W^T: rows (c, k), columns o
        if ((e = disco::launch_transpose_bf16(W->data, wt, (int)Co, (int)CK, sm)) != hipSuccess) return hipfail(e, "W transpose");
        for (int64_t b = 0; b < B; ++b)
            if ((e = disco::launch_transpose_bf16(gyp + b * Co * N, gyt + b * N * Co, (int)Co, (int)N, sm)) != hipSuccess)
                return hipfail(e, "gy transpose");
    }
    // dW partials of chunk c0 (gy times the contraction, over S position splits) and their fixed-order sum
    auto dw_chunk = [&](int64_t c0, int32_t Mc, const uint16_t *outp, int64_t ostride, hipStream_t sd) -> disco_status {
        for (int64_t b = 0; b < B; ++b) {
            disco::GemmNtLaunch g2;
            g2.A = gyp + b * Co * N; g2.lda = N; g2.M = (int32_t)Co; g2.a_bytes = (uint32_t)(Co * N * 2);
            g2.B = outp + b * ostride; g2.ldb = N; g2.N = Mc; g2.b_bytes = (uint32_t)((int64_t)Mc * N * 2);
            g2.Kd = (int32_t)N; g2.k_per_split = L.kps; g2.out_f32 = true;
            g2.C = part + b * (int64_t)L.S * Co * Mc; g2.ldc = Mc; g2.f16 = f16;
            if ((e = disco::launch_gemm_nt(g2, sd)) != hipSuccess) return hipfail(e, "gy out^T product");
        }
        if ((e = disco::launch_reduce_partials(part, (int)(B * L.S), (int)Co, Mc, dW->data, CK, (int)(c0 * K), f16, sd)) !=
            hipSuccess)
            return hipfail(e, "dW reduction");
        return DISCO_OK;
    };
    // With the contraction kept, dW depends on the inputs only: it runs on a second stream, overlapping
    // gx on the caller's stream (ordered by events at both ends).  With gx one fused launch, the
    // recomputed contraction and its dW products likewise run on the second stream beside it (they
    // share no workspace region with it: gbuf and part against wt).  Once the side stream waits on the
    // caller's, every exit joins it back (the guard's destructor on an early error return), so no
    // side-stream work outlives the call unordered.
    struct Fork {
        hipEvent_t in = nullptr, done = nullptr;
        hipStream_t main = nullptr, side = nullptr;  // side set once it waits on `in`
        hipError_t join()
        {
            if (!side) return hipSuccess;
            hipStream_t s = side;
            side = nullptr;
            hipError_t e = hipEventRecord(done, s);
            if (e == hipSuccess) e = hipStreamWaitEvent(main, done, 0);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                (void)hipStreamSynchronize(s);  // cannot order on the device: wait on the host instead
            }
            return e;
        }
        ~Fork()
        {
            (void)join();
            if (in) (void)hipEventDestroy(in);
            if (done) (void)hipEventDestroy(done);
        }
    } fork;
    hipStream_t sd = sm;
    // test knob: DISCO_BWD_OVERLAP=0 keeps the recomputing backward on the caller's stream
    const bool overlap_recompute = gx_fused && !svp && !getenv_is0("DISCO_BWD_OVERLAP");
    if ((svp || overlap_recompute) && C > 0) {
        hipStream_t side = side_stream(h->device);
        fork.main = sm;
        if (side && hipEventCreateWithFlags(&fork.in, hipEventDisableTiming) == hipSuccess &&
            hipEventCreateWithFlags(&fork.done, hipEventDisableTiming) == hipSuccess &&
            hipEventRecord(fork.in, sm) == hipSuccess && hipStreamWaitEvent(side, fork.in, 0) == hipSuccess) {
            sd = side;
            fork.side = side;
        } else {
            (void)hipGetLastError();  // no second stream: everything on the caller's
        }
        for (int64_t c0 = 0; c0 < C && svp; c0 += L.Cc) {
            const int32_t Mc = (int32_t)(std::min<int64_t>(L.Cc, C - c0) * K);
            if ((st = dw_chunk(c0, Mc, svp + c0 * K * N, C * K * N, sd)) != DISCO_OK) return st;
        }
    }
    // the stream of the recomputed contraction and its dW products
    const hipStream_t sc = overlap_recompute ? sd : sm;
    if (gx_fused && C > 0) {
        disco::FusedMfmaLaunch m;
        m.x = gy->data; m.W = wt; m.y = gx->data;
        m.pieces = h->fused_t.pieces; m.rows = h->fused_t.rows; m.descs = h->fused_t.descs;
        m.f16 = f16;
        m.adata = f16 ? h->fused_t.adata16 : h->fused_t.adata;
        m.scale = f16 ? std::ldexp(1.0f, -h->fused_t.psi16_exp) : 1.0f;
        m.ho_piece = h->fused_t.ho_piece; m.ho_order = h->fused_t.ho_order;
        m.B = (int32_t)B; m.C = (int32_t)Co; m.Co = (int32_t)C; m.K = h->K;  // input channels o, output channels c
        m.Ho = h->Hi; m.Wo = h->Wo; m.Hi = h->Ho; m.Wi = h->Wo; m.s = 1;
        m.max_piece_bytes = h->fused_t.max_piece_bytes;
        m.max_resident_bytes = h->fused_t.max_resident_bytes;
        m.desc_bytes = h->fused_t.desc_bytes; m.adata_bytes = h->fused_t.adata_bytes;
        m.w16 = true;  // W' in rows of 16
        if ((e = disco::launch_fused_mfma(m, sm)) != hipSuccess) return hipfail(e, "gx fused");
    }
    for (int64_t c0 = 0; c0 < C; c0 += L.Cc) {
        const int64_t cc = std::min<int64_t>(L.Cc, C - c0);
        const int32_t Mc = (int32_t)(cc * K);
        if (cc <= 0) break;
        if (gx_fused && svp) break;  // gx done, dW on the side stream
        uint16_t *gb = gbuf;  // [b][c k][n] of this chunk
        const int64_t gstride = (int64_t)Mc * N;
        for (int64_t b = 0; b < B && !gx_fused; ++b) {
            // g[c k][n] = sum_o W[o, c0 + c, k] gy[b, o, n]
            disco::GemmNtLaunch g1;
            g1.A = wt + c0 * K * Co; g1.lda = Co; g1.M = Mc; g1.a_bytes = (uint32_t)((int64_t)Mc * Co * 2);
            g1.B = gyt + b * N * Co; g1.ldb = Co; g1.N = (int32_t)N; g1.b_bytes = (uint32_t)(N * Co * 2);
            g1.Kd = (int32_t)Co; g1.k_per_split = 0; g1.out_f32 = false; g1.C = gb + b * gstride; g1.ldc = N;
            g1.f16 = f16;
            if ((e = disco::launch_gemm_nt(g1, sm)) != hipSuccess) return hipfail(e, "W^T gy product");
        }
        // gx[b, c0 + c] = F^T g, every batch in one launch
        if (!gx_fused && (st = enqueue_bwd(h, gb, gxp + c0 * plane_in, dt, B, cc, sm, gstride, C * plane_in)) != DISCO_OK)
            return st;
        // out[b][c k][n] = (F x)[b, c0 + c]: the fused kernel's contraction (psi resident across the
        // chunk's channels) where its plan exists, else the forward contraction; nothing to compute
        // when the caller kept the contraction
        if (svp) {
        } else if (h->fused.ok && !getenv_is0("DISCO_FUSED_MFMA")) {  // test knob: "0" also turns this path off
            disco::FusedContractLaunch m;
            m.x = xp + c0 * plane_in; m.out = gb;
            m.pieces = h->fused.pieces; m.rows = h->fused.rows; m.descs = h->fused.descs;
            m.adata = f16 ? h->fused.adata16 : h->fused.adata;
            m.ho_piece = h->fused.ho_piece; m.ho_order = h->fused.ho_order;
            m.B = (int32_t)B; m.C = (int32_t)cc; m.K = h->K; m.Ho = h->Ho; m.Wo = h->Wo; m.Hi = h->Hi; m.Wi = h->Wi;
            m.s = h->Wi / h->Wo; m.max_piece_bytes = h->fused.max_piece_bytes;
            m.max_resident_bytes = h->fused.max_resident_bytes;
            m.desc_bytes = h->fused.desc_bytes; m.adata_bytes = h->fused.adata_bytes;
            m.f16 = f16; m.scale = f16 ? std::ldexp(1.0f, -h->fused.psi16_exp) : 1.0f;
            m.x_bstride = C * plane_in; m.out_bstride = gstride;
            if ((e = disco::launch_fused_contract(m, sc)) != hipSuccess) return hipfail(e, "contraction");
        } else if ((st = enqueue_fwd(h, xp + c0 * plane_in, gb, dt, B, cc, sc, C * plane_in, gstride)) !=
                   DISCO_OK) {
            return st;
        }
        if (!svp && (st = dw_chunk(c0, Mc, gb, gstride, sc)) != DISCO_OK) return st;
    }
    if ((e = fork.join()) != hipSuccess) return hipfail(e, "side-stream join");
    return DISCO_OK;
}

}  // namespace

disco_status disco_fused_conv_bwd(disco_psi h, const disco_tensor *x, const disco_tensor *W, const disco_tensor *gy,
                                  disco_tensor *gx, disco_tensor *dW, void *workspace, size_t workspace_bytes,
                                  void *stream)
{
    if (!x) return fail(DISCO_ERR_INVALID_ARGUMENT, "x is NULL");
    return fused_conv_bwd_impl(h, x, nullptr, W, gy, gx, dW, workspace, workspace_bytes, stream);
}

disco_status disco_fused_conv_bwd_noalloc(disco_psi h, const disco_tensor *x, const disco_tensor *W,
                                          const disco_tensor *gy, disco_tensor *gx, disco_tensor *dW, void *stream)
{
    disco_status st = check_handle(h);
    if (st != DISCO_OK) return st;
    if (!x) return fail(DISCO_ERR_INVALID_ARGUMENT, "x is NULL");
    void *ws = scratch_ptr(h->device);
    if (!ws) return fail(DISCO_ERR_HIP, "the scratch array of this device was not set up");
    return fused_conv_bwd_impl(h, x, nullptr, W, gy, gx, dW, ws, kScratchBytes, stream, kScratchBytes);
}

disco_status disco_fused_conv_bwd_saved(disco_psi h, const disco_tensor *out, const disco_tensor *W,
                                        const disco_tensor *gy, disco_tensor *gx, disco_tensor *dW, void *workspace,
                                        size_t workspace_bytes, void *stream)
{
    if (!out) return fail(DISCO_ERR_INVALID_ARGUMENT, "out is NULL");
    return fused_conv_bwd_impl(h, nullptr, out, W, gy, gx, dW, workspace, workspace_bytes, stream);
}

}  // extern "C"
