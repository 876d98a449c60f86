// C ABI of the fused int8 convolution library: host-side validation, launch
// dispatch and the bottleneck / network drivers.  Every check runs on the
// host before the first launch, so error paths need no device; the launch
// paths only enqueue kernels on the caller's stream (no allocation, no
// memset, no synchronisation), which also makes them safe to capture into a
// HIP graph.
#include "ifx.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "ifx_internal.h"

namespace ifx {

KernelQuery *&armed_query()
{
    thread_local KernelQuery *q = nullptr;
    return q;
}

}  // namespace ifx

namespace {

thread_local int32_t g_last_hip = 0;

// Arms a kernel-name query for the calling thread for the object's lifetime.
struct ArmedQuery {
    ifx::KernelQuery q;
    ArmedQuery()
    {
        q.name[0] = 0;
        q.answered = false;
        q.even_copy = false;
        ifx::armed_query() = &q;
    }
    ~ArmedQuery() { ifx::armed_query() = nullptr; }
    ArmedQuery(const ArmedQuery &) = delete;
    ArmedQuery &operator=(const ArmedQuery &) = delete;
};

ifx_status copy_name(const ifx::KernelQuery &q, char *buf, size_t len)
{
    if (!q.answered) return IFX_E_UNSUPPORTED;
    const size_t n = strlen(q.name);
    if (n + 1 > len) return IFX_E_WORKSPACE;
    memcpy(buf, q.name, n + 1);
    return IFX_OK;
}

enum Kind { kGeneric, kStem };

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int out_dim(int in, int k, int s, int p)
{
    long long span = (long long)in + 2LL * p - k;
    if (span < 0 || s <= 0) return 0;
    return (int)(span / s + 1);
}

inline int wgroup(int oc)
{
    int r = (oc + 31) / 32 * 32;
    return r < 128 ? r : 128;
}

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t act_bytes(long long n, long long h, long long w, long long c)
{
    if (n <= 0 || h <= 0 || w <= 0 || c <= 0) return 0;
    return (size_t)(n * ((c + 31) / 32) * h * w * 32);
}

struct Dims {
    int ho, wo;   // convolution output
    int oh, ow;   // tensor written (pooled when MAXPOOL)
};

ifx::ConvArgs conv_args(const ifx_conv_desc *d, const Dims &dm, const int8_t *x, const int8_t *w, const int32_t *bias,
                        const int32_t *mult, const int32_t *shift, const int8_t *res, void *y);

ifx_status check_desc(const ifx_conv_desc *d, Kind *kind, Dims *dims)
{
    if (!d) return IFX_E_NULL;
    if (d->n <= 0 || d->h <= 0 || d->w <= 0 || d->c_in <= 0 || d->c_out <= 0 || d->kh <= 0 || d->kw <= 0 ||
        d->stride <= 0 || d->pad < 0)
        return IFX_E_SHAPE;
    const uint32_t f = d->flags;
    if (f & ~(uint32_t)(IFX_RELU | IFX_RESIDUAL | IFX_MAXPOOL | IFX_OUT_I32 | IFX_INPUT_NHWC | IFX_OUT_PHASE |
                        IFX_IN_PHASE))
        return IFX_E_UNSUPPORTED;
    Dims dm;
    dm.ho = out_dim(d->h, d->kh, d->stride, d->pad);
    dm.wo = out_dim(d->w, d->kw, d->stride, d->pad);
    if (dm.ho <= 0 || dm.wo <= 0) return IFX_E_SHAPE;
    dm.oh = dm.ho;
    dm.ow = dm.wo;
    Kind k;
    const int kh = d->kh, kw = d->kw, s = d->stride, p = d->pad;
    if (kh == 7 && kw == 7 && s == 2 && p == 3) {
        if (!(f & IFX_MAXPOOL) || (f & (IFX_RESIDUAL | IFX_OUT_I32))) return IFX_E_UNSUPPORTED;
        if (d->c_in > 4 || d->c_out != 64) return IFX_E_UNSUPPORTED;
        dm.oh = out_dim(dm.ho, 3, 2, 1);
        dm.ow = out_dim(dm.wo, 3, 2, 1);
        if (dm.oh <= 0 || dm.ow <= 0) return IFX_E_SHAPE;
        k = kStem;
    } else if ((kh == 1 && kw == 1 && p == 0 && (s == 1 || s == 2)) ||
               (kh == 3 && kw == 3 && p == 1 && (s == 1 || s == 2))) {
        if (f & (IFX_MAXPOOL | IFX_INPUT_NHWC)) return IFX_E_UNSUPPORTED;
        if ((f & IFX_OUT_I32) && (f & (IFX_RELU | IFX_RESIDUAL))) return IFX_E_UNSUPPORTED;
        if (d->c_out % 4) return IFX_E_UNSUPPORTED;  // per-channel parameters move in 4-channel words
        k = kGeneric;
    } else {
        return IFX_E_UNSUPPORTED;
    }
    // GEMM rows and per-image input planes are indexed with 32-bit integers
    if ((long long)d->n * dm.ho * dm.wo > 0x7fffffffLL || (long long)d->n * d->h * d->w > 0x7fffffffLL ||
        (long long)d->c_out * 16 > 0x7fffffffLL)
        return IFX_E_SHAPE;
    if (f & (IFX_OUT_PHASE | IFX_IN_PHASE)) {  // the general kernel's phase-split layout
        if (k != kGeneric) return IFX_E_UNSUPPORTED;
        const ifx::ConvArgs a = conv_args(d, dm, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
        if (!ifx::conv_phase_supported(a, kh, kw)) return IFX_E_UNSUPPORTED;
    }
    if (kind) *kind = k;
    if (dims) *dims = dm;
    return IFX_OK;
}

ifx_status hip_status(hipError_t e)
{
    if (e == hipSuccess) return IFX_OK;
    g_last_hip = (int32_t)e;
    return IFX_E_HIP;
}

ifx::ConvArgs conv_args(const ifx_conv_desc *d, const Dims &dm, const int8_t *x, const int8_t *w, const int32_t *bias,
                        const int32_t *mult, const int32_t *shift, const int8_t *res, void *y);

// Launch one validated convolution.
ifx_status run_conv(const ifx_conv_desc *d, Kind kind, const Dims &dm, const int8_t *x, const int8_t *w,
                    const int32_t *bias, const int32_t *mult, const int32_t *shift, const int8_t *res, void *y,
                    hipStream_t s, int32_t *part = nullptr, size_t part_bytes = 0)
{
    if (kind == kStem) {
        ifx::StemArgs a;
        a.x = x;
        a.wt = w;
        a.bias = bias;
        a.mult = mult;
        a.shift = shift;
        a.y = (int8_t *)y;
        a.n = d->n;
        a.h = d->h;
        a.w = d->w;
        a.c = d->c_in;
        a.nhwc = (d->flags & IFX_INPUT_NHWC) ? 1 : 0;
        a.ho = dm.ho;
        a.wo = dm.wo;
        a.ph = dm.oh;
        a.pw = dm.ow;
        a.relu = (d->flags & IFX_RELU) ? 1 : 0;
        return hip_status(ifx::launch_stem(a, s));
    }
    return hip_status(
        ifx::launch_conv_split(conv_args(d, dm, x, w, bias, mult, shift, res, y), d->kh, d->kw, part, part_bytes, s));
}

// Partial-sum bytes run_conv may use for a validated non-stem convolution (split-K).
size_t conv_part_bytes(const ifx_conv_desc *d, const Dims &dm)
{
    return ifx::splitk_bytes(conv_args(d, dm, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), d->kh,
                             d->kw);
}

// Kernel arguments of a validated non-stem convolution.
ifx::ConvArgs conv_args(const ifx_conv_desc *d, const Dims &dm, const int8_t *x, const int8_t *w, const int32_t *bias,
                        const int32_t *mult, const int32_t *shift, const int8_t *res, void *y)
{
    ifx::ConvArgs a;
    a.x = x;
    a.wt = w;
    a.bias = bias;
    a.mult = mult;
    a.shift = shift;
    a.res = res;
    a.y = y;
    a.n = d->n;
    a.h = d->h;
    a.w = d->w;
    a.i1 = (d->c_in + 31) / 32;
    a.ho = dm.ho;
    a.wo = dm.wo;
    a.oc = d->c_out;
    a.oc1 = (d->c_out + 31) / 32;
    a.o2 = wgroup(d->c_out);
    a.stride = d->stride;
    a.pad = d->pad;
    a.m = d->n * dm.ho * dm.wo;
    a.nkb = d->kh * d->kw * a.i1;
    a.relu = (d->flags & IFX_RELU) ? 1 : 0;
    a.residual = (d->flags & IFX_RESIDUAL) ? 1 : 0;
    a.out_i32 = (d->flags & IFX_OUT_I32) ? 1 : 0;
    a.out_even = 0;
    a.y_even = nullptr;
    a.in_ps = (d->flags & IFX_IN_PHASE) ? 1 : 0;
    a.out_ps = (d->flags & IFX_OUT_PHASE) ? 1 : 0;
    a.ksplit = 1;
    a.kb_per = 0;
    ifx::fastdiv_magic((unsigned)(dm.ho * dm.wo), &a.howo_mul, &a.howo_shr);
    ifx::fastdiv_magic((unsigned)dm.wo, &a.wo_mul, &a.wo_shr);
    ifx::fastdiv_magic((unsigned)a.o2, &a.o2_mul, &a.o2_shr);
    return a;
}

// The network driver's rule too: the kernel that runs d (with split-K partial sums of part_bytes
// available) writes an even-pixel copy.
bool even_copy_ok(const ifx_conv_desc *d, const Dims &dm, int32_t *part, size_t part_bytes)
{
    if (d->flags & (IFX_OUT_I32 | IFX_OUT_PHASE | IFX_MAXPOOL)) return false;
    ArmedQuery aq;
    if (hip_status(ifx::launch_conv_split(conv_args(d, dm, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                    nullptr),
                                          d->kh, d->kw, part, part_bytes, nullptr)) != IFX_OK)
        return false;
    return aq.q.answered && aq.q.even_copy;
}

ifx_status check_conv_ptrs(const ifx_conv_desc *d, const int8_t *x, const int8_t *w, const int32_t *bias,
                           const int32_t *mult, const int32_t *shift, const int8_t *res, const void *y)
{
    const bool i32 = (d->flags & IFX_OUT_I32) != 0;
    if (!x || !w || !bias || !y) return IFX_E_NULL;
    if (!i32 && (!mult || !shift)) return IFX_E_NULL;
    if ((d->flags & IFX_RESIDUAL) && !res) return IFX_E_NULL;
    if (!aligned16(x) || !aligned16(w) || !aligned16(bias) || !aligned16(y)) return IFX_E_ALIGN;
    if (!i32 && (!aligned16(mult) || !aligned16(shift))) return IFX_E_ALIGN;
    if ((d->flags & IFX_RESIDUAL) && !aligned16(res)) return IFX_E_ALIGN;
    return IFX_OK;
}

// ---- bottleneck ----

struct BlockPlan {
    Kind kind[4];
    Dims dims[4];
    size_t t1, t2, sc;  // workspace pieces (bytes, 256-aligned)
    size_t part;        // split-K partial sums (bytes, 256-aligned; 0 when no conv splits)
};

bool flags_plain(uint32_t f) { return (f & (IFX_RESIDUAL | IFX_MAXPOOL | IFX_OUT_I32)) == 0; }
bool proj_fusable(const ifx_conv_desc *d3, const ifx_conv_desc *dp);

// Validate the block's descriptors for batch n (n <= 0: use d[0].n) and their chaining.
ifx_status plan_block(const ifx_block_params *p, int n, BlockPlan *plan)
{
    if (!p) return IFX_E_NULL;
    ifx_conv_desc d[4];
    const int nd = p->has_proj ? 4 : 3;
    for (int i = 0; i < nd; ++i) {
        d[i] = p->d[i];
        if (n > 0) d[i].n = n;
    }
    for (int i = 0; i < nd; ++i) {
        ifx_status st = check_desc(&d[i], &plan->kind[i], &plan->dims[i]);
        if (st != IFX_OK) return st;
        if (plan->kind[i] != kGeneric) return IFX_E_UNSUPPORTED;
        if (d[i].flags & IFX_OUT_I32) return IFX_E_UNSUPPORTED;
    }
    for (int i = 0; i < nd; ++i)  // layouts between a block's convolutions are the driver's choice
        if (d[i].flags & (IFX_OUT_PHASE | IFX_IN_PHASE)) return IFX_E_UNSUPPORTED;
    if (!flags_plain(d[0].flags) || !flags_plain(d[1].flags)) return IFX_E_UNSUPPORTED;
    if (!(d[2].flags & IFX_RESIDUAL) || (d[2].flags & (IFX_MAXPOOL | IFX_OUT_I32))) return IFX_E_UNSUPPORTED;
    if (p->has_proj && !flags_plain(d[3].flags)) return IFX_E_UNSUPPORTED;
    const Dims &a = plan->dims[0], &b = plan->dims[1], &c = plan->dims[2];
    if (d[1].n != d[0].n || d[2].n != d[0].n) return IFX_E_SHAPE;
    if (d[1].c_in != d[0].c_out || d[1].h != a.oh || d[1].w != a.ow) return IFX_E_SHAPE;
    if (d[2].c_in != d[1].c_out || d[2].h != b.oh || d[2].w != b.ow) return IFX_E_SHAPE;
    if (p->has_proj) {
        const Dims &q = plan->dims[3];
        if (d[3].n != d[0].n || d[3].c_in != d[0].c_in || d[3].h != d[0].h || d[3].w != d[0].w) return IFX_E_SHAPE;
        if (d[3].c_out != d[2].c_out || q.oh != c.oh || q.ow != c.ow) return IFX_E_SHAPE;
    } else {
        if (d[2].c_out != d[0].c_in || c.oh != d[0].h || c.ow != d[0].w) return IFX_E_SHAPE;
    }
    plan->t1 = round_up(act_bytes(d[0].n, a.oh, a.ow, d[0].c_out), 256);
    plan->t2 = round_up(act_bytes(d[1].n, b.oh, b.ow, d[1].c_out), 256);
    plan->sc = p->has_proj ? round_up(act_bytes(d[3].n, plan->dims[3].oh, plan->dims[3].ow, d[3].c_out), 256) : 0;
    // split-K partial sums of c1, c2 and the conv3 / projection that do not run fused
    plan->part = std::max(conv_part_bytes(&d[0], plan->dims[0]), conv_part_bytes(&d[1], plan->dims[1]));
    if (!(p->has_proj && proj_fusable(&d[2], &d[3]))) {
        plan->part = std::max(plan->part, conv_part_bytes(&d[2], plan->dims[2]));
        if (p->has_proj) plan->part = std::max(plan->part, conv_part_bytes(&d[3], plan->dims[3]));
    }
    return IFX_OK;
}

ifx_status check_block_ptrs(const ifx_block_params *p)
{
    const int nd = p->has_proj ? 4 : 3;
    for (int i = 0; i < nd; ++i) {
        if (!p->w_blk[i] || !p->bias[i] || !p->mult[i] || !p->shift[i]) return IFX_E_NULL;
        if (!aligned16(p->w_blk[i]) || !aligned16(p->bias[i]) || !aligned16(p->mult[i]) || !aligned16(p->shift[i]))
            return IFX_E_ALIGN;
    }
    return IFX_OK;
}

// A conv3 / projection pair that ifx_conv_proj_fused computes (descriptors already valid and chained).
bool proj_fusable(const ifx_conv_desc *d3, const ifx_conv_desc *dp)
{
    return d3->kh == 1 && d3->kw == 1 && d3->stride == 1 && d3->pad == 0 && dp->kh == 1 && dp->kw == 1 &&
           dp->pad == 0 && (d3->flags & ~(uint32_t)IFX_RELU) == IFX_RESIDUAL && dp->flags == 0;
}

// A conv3 (with its shortcut) and the next block's conv1 that ifx_conv_chain_fused computes in one
// launch (descriptors already valid; both at the same batch).
bool chain_fusable(const ifx_conv_desc *d3, const Dims &m3, const ifx_conv_desc *d1, const Dims &m1)
{
    if (d3->kh != 1 || d3->kw != 1 || d3->stride != 1 || d3->pad != 0) return false;
    if (d1->kh != 1 || d1->kw != 1 || d1->stride != 1 || d1->pad != 0) return false;
    if (d3->flags != (IFX_RESIDUAL | IFX_RELU) || (d1->flags & ~(uint32_t)(IFX_RELU | IFX_OUT_PHASE))) return false;
    if (d1->n != d3->n || d1->h != m3.oh || d1->w != m3.ow || d1->c_in != d3->c_out) return false;
    const ifx::ConvArgs a = conv_args(d3, m3, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    const ifx::ConvArgs b = conv_args(d1, m1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    return ifx::conv1x1_chain_supported(a, b);
}

// A block whose input is read only by its conv1 and by a stride-2 1x1 projection: when the
// previous block chains this conv1, it needs to store only the input's even rows and columns.
bool reads_input_even(const ifx_block_params *p)
{
    const ifx_conv_desc &pj = p->d[3];
    return p->has_proj && pj.kh == 1 && pj.kw == 1 && pj.stride == 2 && pj.pad == 0;
}

// A conv3 with its projection (proj_fusable) and the next block's conv1 that
// ifx_conv_proj_chain_fused computes in one launch (descriptors already valid).
bool proj_chain_fusable(const ifx_conv_desc *d3, const Dims &m3, const ifx_conv_desc *dp, const Dims &mp,
                        const ifx_conv_desc *d1, const Dims &m1)
{
    if (!chain_fusable(d3, m3, d1, m1)) return false;
    const ifx::ConvArgs a = conv_args(d3, m3, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    const ifx::ConvArgs pj = conv_args(dp, mp, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    const ifx::ConvArgs b = conv_args(d1, m1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    return ifx::conv1x1_proj_chain_supported(a, pj, b);
}

// How one block of a network hands data to the next.  In (for this block): its conv1 output is
// already in t1 (the previous block chained it), possibly phase-split, and its input x holds only
// the even pixels.  Out (for the next block): the same three facts about what this block left.
struct BlockFlow {
    bool have_t1 = false, t1_ps = false, x_even = false;
    const int8_t *xe = nullptr;  // or: the block input's even pixels, densely (its projection's input)
};

// A stride-2 pad-1 3x3 on even sizes whose kernel reads the phase-split layout.
bool phase_in_ok(const ifx_conv_desc &d)
{
    if (!(d.kh == 3 && d.kw == 3 && d.stride == 2 && d.pad == 1 && !(d.h & 1) && !(d.w & 1))) return false;
    ifx_conv_desc q = d;
    q.flags |= IFX_IN_PHASE;
    return check_desc(&q, nullptr, nullptr) == IFX_OK;
}

// The same convolution as a launch of its own writing the phase-split layout.
bool phase_out_ok(const ifx_conv_desc &d)
{
    ifx_conv_desc q = d;
    q.flags |= IFX_OUT_PHASE;
    return check_desc(&q, nullptr, nullptr) == IFX_OK;
}

// Launch a validated block for batch n; workspace already checked.  `in` describes what the
// previous block left (see BlockFlow).  next (or null): the following block; when this block's
// conv3 chains with next's conv1, both run as one launch that also leaves next's t1 in the
// workspace (phase-split when next's conv2 reads it so), and y receives only the even pixels if
// next reads its input only through its conv1 and a stride-2 projection; *out says so.  When this
// block's conv3 runs alone and next has such a projection (fused), the conv3 kernel also writes
// y's even pixels into the workspace's shortcut region, where next's projection reads them with
// unit stride (out->xe).
ifx_status run_block(const ifx_block_params *p, const BlockPlan &plan, int n, const int8_t *x, int8_t *y,
                     int8_t *ws, int32_t *part, size_t part_bytes, hipStream_t s, const BlockFlow &in = BlockFlow(),
                     const ifx_block_params *next = nullptr, BlockFlow *out = nullptr)
{
    ifx_conv_desc d[4];
    const int nd = p->has_proj ? 4 : 3;
    for (int i = 0; i < nd; ++i) {
        d[i] = p->d[i];
        d[i].n = n;
    }
    if (out) *out = BlockFlow();
    if ((in.x_even && !in.have_t1) || ((in.x_even || in.xe) && !reads_input_even(p))) return IFX_E_UNSUPPORTED;
    if (in.x_even || in.xe) {
        d[3].stride = 1;  // the same output pixels, read from the subsampled input
        d[3].h = (d[3].h + 1) / 2;
        d[3].w = (d[3].w + 1) / 2;
    }
    const int8_t *const px = in.xe ? in.xe : x;  // the projection's input
    // t1 between conv1 and a stride-2 conv2 goes phase-split when both kernels handle it
    bool t1_ps;
    if (in.have_t1) {
        t1_ps = in.t1_ps;
    } else {
        t1_ps = phase_in_ok(d[1]) && phase_out_ok(d[0]);
        if (t1_ps) d[0].flags |= IFX_OUT_PHASE;
    }
    if (t1_ps) d[1].flags |= IFX_IN_PHASE;
    int8_t *t1 = ws;
    int8_t *t2 = ws + plan.t1;
    int8_t *sc = ws + plan.t1 + plan.t2;
    ifx_status st;
    if (!in.have_t1) {
        st = run_conv(&d[0], kGeneric, plan.dims[0], x, p->w_blk[0], p->bias[0], p->mult[0], p->shift[0], nullptr, t1,
                      s, part, part_bytes);
        if (st != IFX_OK) return st;
    }
    st = run_conv(&d[1], kGeneric, plan.dims[1], t1, p->w_blk[1], p->bias[1], p->mult[1], p->shift[1], nullptr, t2, s,
                  part, part_bytes);
    if (st != IFX_OK) return st;
    // next's conv1 descriptor when this block could chain it (phase-split for a stride-2 conv2)
    ifx_conv_desc d1;
    Dims m1;
    bool can_chain = false;
    if (next) {
        d1 = next->d[0];
        d1.n = n;
        can_chain = check_desc(&d1, nullptr, &m1) == IFX_OK;
        if (can_chain) {
            ifx_conv_desc nd1 = next->d[1];
            nd1.n = n;
            if (phase_in_ok(nd1)) d1.flags |= IFX_OUT_PHASE;
        }
    }
    const int8_t *res = x;
    if (p->has_proj && can_chain && proj_fusable(&d[2], &d[3]) &&
        proj_chain_fusable(&d[2], plan.dims[2], &d[3], plan.dims[3], &d1, m1)) {
        // conv3, its projection and the next block's conv1 in one launch
        const ifx::ConvArgs a = conv_args(&d[2], plan.dims[2], t2, p->w_blk[2], p->bias[2], p->mult[2], p->shift[2],
                                          nullptr, y);
        const ifx::ConvArgs pj = conv_args(&d[3], plan.dims[3], px, p->w_blk[3], p->bias[3], p->mult[3],
                                           p->shift[3], nullptr, nullptr);
        const ifx::ConvArgs b = conv_args(&d1, m1, y, next->w_blk[0], next->bias[0], next->mult[0], next->shift[0],
                                          nullptr, t1);
        st = hip_status(ifx::launch_conv1x1_proj_chain(a, pj, b, s));
        if (st == IFX_OK && out) {
            out->have_t1 = true;
            out->t1_ps = b.out_ps != 0;
        }
        return st;
    }
    if (p->has_proj) {
        if (proj_fusable(&d[2], &d[3])) {
            // conv3 and the projection in one kernel: the shortcut never goes through HBM
            const ifx::ConvArgs a = conv_args(&d[2], plan.dims[2], t2, p->w_blk[2], p->bias[2], p->mult[2],
                                              p->shift[2], nullptr, y);
            const ifx::ConvArgs pj = conv_args(&d[3], plan.dims[3], px, p->w_blk[3], p->bias[3], p->mult[3],
                                               p->shift[3], nullptr, nullptr);
            return hip_status(ifx::launch_conv_proj(a, pj, s));
        }
        if (in.xe) return IFX_E_UNSUPPORTED;  // the shortcut region holds the projection's input
        st = run_conv(&d[3], kGeneric, plan.dims[3], x, p->w_blk[3], p->bias[3], p->mult[3], p->shift[3], nullptr,
                      sc, s, part, part_bytes);
        if (st != IFX_OK) return st;
        res = sc;
    } else if (can_chain && chain_fusable(&d[2], plan.dims[2], &d1, m1)) {
        // conv3 and the next block's conv1 in one launch: the block output is read from LDS
        ifx::ConvArgs a = conv_args(&d[2], plan.dims[2], t2, p->w_blk[2], p->bias[2], p->mult[2], p->shift[2], x, y);
        const bool even = reads_input_even(next);
        a.out_even = even ? 1 : 0;
        const ifx::ConvArgs b = conv_args(&d1, m1, y, next->w_blk[0], next->bias[0], next->mult[0], next->shift[0],
                                          nullptr, t1);
        st = hip_status(ifx::launch_conv1x1_chain(a, b, s));
        if (st == IFX_OK && out) {
            out->have_t1 = true;
            out->t1_ps = b.out_ps != 0;
            out->x_even = even;
        }
        return st;
    }
    if (next && out && !p->has_proj && reads_input_even(next)) {
        // next's projection, fused, reading this output's even pixels from the shortcut region
        ifx_conv_desc n2 = next->d[2], n3 = next->d[3];
        n2.n = n3.n = n;
        n3.stride = 1;
        const Dims &m2 = plan.dims[2];
        const size_t even_bytes = act_bytes(n, (m2.ho + 1) / 2, (m2.wo + 1) / 2, d[2].c_out);
        if (proj_fusable(&n2, &n3) && even_bytes <= plan.sc && even_copy_ok(&d[2], m2, part, part_bytes)) {
            ifx::ConvArgs a = conv_args(&d[2], m2, t2, p->w_blk[2], p->bias[2], p->mult[2], p->shift[2], res, y);
            a.y_even = sc;
            st = hip_status(ifx::launch_conv_split(a, d[2].kh, d[2].kw, part, part_bytes, s));
            if (st == IFX_OK) out->xe = sc;
            return st;
        }
    }
    return run_conv(&d[2], kGeneric, plan.dims[2], t2, p->w_blk[2], p->bias[2], p->mult[2], p->shift[2], res, y, s,
                    part, part_bytes);
}

// ---- network ----

struct NetPlan {
    Kind stem_kind;
    Dims stem_dims;
    size_t act, t1, t2, sc, pool;  // workspace pieces for batch nb
    size_t part;                   // split-K partial sums (max over the network's convolutions)
    int out_h, out_w, out_c;       // backbone output
    int nb;                        // images per pass
    int lanes;                     // passes in flight at once, each with its own workspace
};

// Library-held block workspace for callers that cannot allocate (ifx_block_forward_noalloc).
// Each device holds its own copy for the life of the process.  In host code the name is a
// host-side stand-in, never a device address: kernels get the address scratch_ptr() looked up.
static __device__ __align__(256) int8_t scratch[IFX_BLOCK_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up once per device (with that
// device current) and kept.
hipError_t scratch_ptr(int8_t **out)
{
    static std::mutex mu;
    static std::vector<int8_t *> ptrs;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> g(mu);
    if ((size_t)dev >= ptrs.size()) ptrs.resize(dev + 1, nullptr);
    if (!ptrs[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        ptrs[dev] = (int8_t *)p;
    }
    *out = ptrs[dev];
    return hipSuccess;
}

// A whole batch of at least this many images (sub_batch 0) runs as two concurrent halves, one on
// the caller's stream and one on a library stream: the last, partly filled round of tiles of
// each launch then overlaps the other half's work.
constexpr int kTwoLaneMin = 192;

ifx_status plan_net(const ifx_net_params *p, int n, NetPlan *plan)
{
    if (!p) return IFX_E_NULL;
    if (n <= 0 || p->n_blocks < 0 || p->sub_batch < 0 || p->fc_in <= 0 || p->fc_out <= 0) return IFX_E_SHAPE;
    if (p->n_blocks > 0 && !p->blocks) return IFX_E_NULL;
    const bool halves = p->sub_batch == 0 && n >= kTwoLaneMin;
    const int nb = halves ? (n + 1) / 2 : (p->sub_batch > 0 && p->sub_batch < n) ? p->sub_batch : n;
    plan->nb = nb;
    plan->lanes = halves ? 2 : 1;
    ifx_conv_desc stem = p->stem;
    stem.n = nb;
    ifx_status st = check_desc(&stem, &plan->stem_kind, &plan->stem_dims);
    if (st != IFX_OK) return st;
    if (plan->stem_kind != kStem) return IFX_E_UNSUPPORTED;
    int h = plan->stem_dims.oh, w = plan->stem_dims.ow, c = stem.c_out;
    size_t act = act_bytes(nb, h, w, c), t1 = 0, t2 = 0, sc = 0, part = 0;
    for (int i = 0; i < p->n_blocks; ++i) {
        const ifx_block_params &bp = p->blocks[i];
        if (bp.d[0].c_in != c || bp.d[0].h != h || bp.d[0].w != w) return IFX_E_SHAPE;
        BlockPlan b;
        st = plan_block(&bp, nb, &b);
        if (st != IFX_OK) return st;
        t1 = std::max(t1, b.t1);
        t2 = std::max(t2, b.t2);
        sc = std::max(sc, b.sc);
        part = std::max(part, b.part);
        h = b.dims[2].oh;
        w = b.dims[2].ow;
        c = bp.d[2].c_out;
        act = std::max(act, act_bytes(nb, h, w, c));
    }
    if (c != p->fc_in) return IFX_E_SHAPE;
    if ((long long)nb * p->fc_out > 0x7fffffffLL) return IFX_E_SHAPE;
    plan->out_h = h;
    plan->out_w = w;
    plan->out_c = c;
    plan->act = round_up(act, 256);
    plan->t1 = t1;
    plan->t2 = t2;
    plan->sc = sc;
    plan->pool = round_up(act_bytes(nb, 1, 1, c), 256);
    ifx_conv_desc fd = {nb, 1, 1, p->fc_in, p->fc_out, 1, 1, 1, 0, IFX_OUT_I32};
    Kind fk;
    Dims fdm;
    if (check_desc(&fd, &fk, &fdm) == IFX_OK) part = std::max(part, conv_part_bytes(&fd, fdm));
    plan->part = part;
    return IFX_OK;
}

size_t lane_ws_bytes(const NetPlan &pl) { return 2 * pl.act + pl.t1 + pl.t2 + pl.sc + pl.pool + pl.part; }
size_t net_ws_bytes(const NetPlan &pl) { return pl.lanes * lane_ws_bytes(pl); }

// The second lane of a two-pass batch: a stream plus the events that fork it from the caller's
// stream and join it back.
struct Lane {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};

hipError_t make_lane(Lane *l)
{
    hipError_t e = hipStreamCreateWithFlags(&l->stream, hipStreamNonBlocking);  // default priority
    if (e == hipSuccess) e = hipEventCreateWithFlags(&l->fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&l->join, hipEventDisableTiming);
    return e;
}

void free_lane(Lane *l)
{
    if (l->fork) (void)hipEventDestroy(l->fork);
    if (l->join) (void)hipEventDestroy(l->join);
    if (l->stream) (void)hipStreamDestroy(l->stream);
    *l = Lane();
}

// The library's lane on the current device, created on first use and kept for the process.
// Callers hold lane_mutex() around the fork (record + wait) and around the join, so two host
// threads never interleave on one event; their second-lane work is serialised on the stream.
std::mutex &lane_mutex()
{
    static std::mutex mu;
    return mu;
}

hipError_t device_lane(Lane *out)
{
    static std::vector<Lane> lanes;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if ((size_t)dev >= lanes.size()) lanes.resize(dev + 1);
    if (!lanes[dev].stream) {
        Lane l;
        e = make_lane(&l);
        if (e != hipSuccess) {
            free_lane(&l);
            return e;
        }
        lanes[dev] = l;
    }
    *out = lanes[dev];
    return hipSuccess;
}

// Validation shared by ifx_conv_chain_fused and its name query.  *d3c receives d3 without
// IFX_OUT_EVEN (a flag of this call only) and *even whether it was set.
ifx_status check_chain(const ifx_conv_desc *d3, const ifx_conv_desc *d1, Dims *m3, Dims *m1, ifx_conv_desc *d3c,
                       bool *even)
{
    if (!d3 || !d1) return IFX_E_NULL;
    *d3c = *d3;
    *even = (d3->flags & IFX_OUT_EVEN) != 0;
    d3c->flags &= ~(uint32_t)IFX_OUT_EVEN;
    Kind k3, k1;
    ifx_status st = check_desc(d3c, &k3, m3);
    if (st != IFX_OK) return st;
    st = check_desc(d1, &k1, m1);
    if (st != IFX_OK) return st;
    if (k3 != kGeneric || k1 != kGeneric) return IFX_E_UNSUPPORTED;
    if (d1->n != d3c->n || d1->h != m3->oh || d1->w != m3->ow || d1->c_in != d3c->c_out) return IFX_E_SHAPE;
    if (!chain_fusable(d3c, *m3, d1, *m1)) return IFX_E_UNSUPPORTED;
    return IFX_OK;
}

// Validation shared by ifx_conv_proj_chain_fused and its name query.
ifx_status check_proj_chain(const ifx_conv_desc *d3, const ifx_conv_desc *dp, const ifx_conv_desc *d1, Dims *m3,
                            Dims *mp, Dims *m1)
{
    if (!d3 || !dp || !d1) return IFX_E_NULL;
    Kind k3, kp, k1;
    ifx_status st = check_desc(d3, &k3, m3);
    if (st == IFX_OK) st = check_desc(dp, &kp, mp);
    if (st == IFX_OK) st = check_desc(d1, &k1, m1);
    if (st != IFX_OK) return st;
    if (k3 != kGeneric || kp != kGeneric || k1 != kGeneric) return IFX_E_UNSUPPORTED;
    if (dp->n != d3->n || dp->c_out != d3->c_out || mp->oh != m3->oh || mp->ow != m3->ow) return IFX_E_SHAPE;
    if (d1->n != d3->n || d1->h != m3->oh || d1->w != m3->ow || d1->c_in != d3->c_out) return IFX_E_SHAPE;
    if (!proj_fusable(d3, dp) || !proj_chain_fusable(d3, *m3, dp, *mp, d1, *m1)) return IFX_E_UNSUPPORTED;
    return IFX_OK;
}

}  // namespace

extern "C" {

ifx_status ifx_conv_validate(const ifx_conv_desc *d) { return check_desc(d, nullptr, nullptr); }

ifx_status ifx_conv_out_dims(const ifx_conv_desc *d, int32_t *ho, int32_t *wo)
{
    Dims dm;
    ifx_status st = check_desc(d, nullptr, &dm);
    if (st != IFX_OK) return st;
    if (!ho || !wo) return IFX_E_NULL;
    *ho = dm.oh;
    *wo = dm.ow;
    return IFX_OK;
}

size_t ifx_act_bytes(int32_t n, int32_t h, int32_t w, int32_t c) { return act_bytes(n, h, w, c); }

size_t ifx_wpack_bytes(const ifx_conv_desc *d)
{
    Kind k;
    if (check_desc(d, &k, nullptr) != IFX_OK) return 0;
    if (k == kStem) return (size_t)d->c_out * 256;
    const int o2 = wgroup(d->c_out);
    const size_t o1 = (size_t)(d->c_out + o2 - 1) / o2;
    return o1 * d->kh * d->kw * ((d->c_in + 31) / 32) * o2 * 32;
}

ifx_status ifx_pack_act(const int8_t *x_nhwc, int8_t *x_blk, int32_t n, int32_t h, int32_t w, int32_t c,
                        void *stream)
{
    if (!x_nhwc || !x_blk) return IFX_E_NULL;
    if (n <= 0 || h <= 0 || w <= 0 || c <= 0 || (long long)n * h * w > 0x7fffffffLL) return IFX_E_SHAPE;
    if (!aligned16(x_blk)) return IFX_E_ALIGN;
    return hip_status(ifx::launch_pack_act(x_nhwc, x_blk, n, h, w, c, (hipStream_t)stream));
}

ifx_status ifx_quantize_f32(const float *x, int8_t *q, int64_t count, int32_t c, const float *mult, void *stream)
{
    if (!x || !q || !mult) return IFX_E_NULL;
    if (c < 1 || count < 0 || count > 0x7fffffffLL || count % c) return IFX_E_SHAPE;
    if (!aligned16(x) || !aligned16(q) || (reinterpret_cast<uintptr_t>(mult) & 3u)) return IFX_E_ALIGN;
    if (count == 0) return IFX_OK;
    return hip_status(ifx::launch_quantize(x, false, q, (int)count, c, nullptr, mult, (hipStream_t)stream));
}

ifx_status ifx_quantize_u8(const uint8_t *x, int8_t *q, int64_t count, int32_t c, const float *mean,
                           const float *mult, void *stream)
{
    if (!x || !q || !mean || !mult) return IFX_E_NULL;
    if (c < 1 || count < 0 || count > 0x7fffffffLL || count % c) return IFX_E_SHAPE;
    if (!aligned16(x) || !aligned16(q) || (reinterpret_cast<uintptr_t>(mean) & 3u) ||
        (reinterpret_cast<uintptr_t>(mult) & 3u))
        return IFX_E_ALIGN;
    if (count == 0) return IFX_OK;
    return hip_status(ifx::launch_quantize(x, true, q, (int)count, c, mean, mult, (hipStream_t)stream));
}

ifx_status ifx_dequantize_i32(const int32_t *q, float *y, int64_t count, float scale, void *stream)
{
    if (!q || !y) return IFX_E_NULL;
    if (count < 0 || count > 0x7fffffffLL) return IFX_E_SHAPE;
    if (!aligned16(q) || !aligned16(y)) return IFX_E_ALIGN;
    if (count == 0) return IFX_OK;
    return hip_status(ifx::launch_dequantize(q, y, (int)count, scale, (hipStream_t)stream));
}

ifx_status ifx_unpack_act(const int8_t *x_blk, int8_t *x_nhwc, int32_t n, int32_t h, int32_t w, int32_t c,
                          void *stream)
{
    if (!x_nhwc || !x_blk) return IFX_E_NULL;
    if (n <= 0 || h <= 0 || w <= 0 || c <= 0 || (long long)n * h * w > 0x7fffffffLL) return IFX_E_SHAPE;
    if (!aligned16(x_blk)) return IFX_E_ALIGN;
    return hip_status(ifx::launch_unpack_act(x_blk, x_nhwc, n, h, w, c, (hipStream_t)stream));
}

ifx_status ifx_pack_weights(const ifx_conv_desc *d, const int8_t *w_ohwi, int8_t *w_blk, void *stream)
{
    Kind k;
    ifx_status st = check_desc(d, &k, nullptr);
    if (st != IFX_OK) return st;
    if (!w_ohwi || !w_blk) return IFX_E_NULL;
    if (!aligned16(w_blk)) return IFX_E_ALIGN;
    hipStream_t s = (hipStream_t)stream;
    if (k == kStem) return hip_status(ifx::launch_pack_weights_stem(w_ohwi, w_blk, d->c_out, d->c_in, s));
    return hip_status(ifx::launch_pack_weights(w_ohwi, w_blk, d->c_out, d->kh, d->kw, d->c_in, wgroup(d->c_out), s));
}

ifx_status ifx_fold_bn(const ifx_bn_fold *f, int32_t *bias, int32_t *mult, int32_t *shift, int32_t *status,
                       void *stream)
{
    if (!f) return IFX_E_NULL;
    if (f->c_out <= 0) return IFX_E_SHAPE;
    if (!f->w_scale || !f->gamma || !f->beta || !f->mean || !f->var || !bias || !mult || !shift || !status)
        return IFX_E_NULL;
    const void *words[] = {f->w_scale, f->gamma, f->beta, f->mean, f->var, status};
    for (const void *p : words)
        if (reinterpret_cast<uintptr_t>(p) & 3u) return IFX_E_ALIGN;
    if (f->conv_bias && (reinterpret_cast<uintptr_t>(f->conv_bias) & 3u)) return IFX_E_ALIGN;
    if (!aligned16(bias) || !aligned16(mult) || !aligned16(shift)) return IFX_E_ALIGN;
    ifx::FoldArgs a;
    a.c_out = f->c_out;
    a.x_scale = f->x_scale;
    a.y_scale = f->y_scale;
    a.eps = f->eps;
    a.w_per_channel = f->w_per_channel ? 1 : 0;
    a.w_scale = f->w_scale;
    a.conv_bias = f->conv_bias;
    a.gamma = f->gamma;
    a.beta = f->beta;
    a.mean = f->mean;
    a.var = f->var;
    return hip_status(ifx::launch_fold_bn(a, bias, mult, shift, status, (hipStream_t)stream));
}

ifx_status ifx_conv_fused(const ifx_conv_desc *d, const int8_t *x_blk, const int8_t *w_blk, const int32_t *bias,
                          const int32_t *mult, const int32_t *shift, const int8_t *residual, void *y, void *stream)
{
    Kind k;
    Dims dm;
    ifx_status st = check_desc(d, &k, &dm);
    if (st != IFX_OK) return st;
    st = check_conv_ptrs(d, x_blk, w_blk, bias, mult, shift, residual, y);
    if (st != IFX_OK) return st;
    return run_conv(d, k, dm, x_blk, w_blk, bias, mult, shift, (d->flags & IFX_RESIDUAL) ? residual : nullptr, y,
                    (hipStream_t)stream);
}

ifx_status ifx_conv_fused_even(const ifx_conv_desc *d, const int8_t *x_blk, const int8_t *w_blk, const int32_t *bias,
                               const int32_t *mult, const int32_t *shift, const int8_t *residual, void *y,
                               int8_t *y_even, void *stream)
{
    Kind k;
    Dims dm;
    ifx_status st = check_desc(d, &k, &dm);
    if (st != IFX_OK) return st;
    st = check_conv_ptrs(d, x_blk, w_blk, bias, mult, shift, residual, y);
    if (st != IFX_OK) return st;
    if (!y_even) return IFX_E_NULL;
    if (!aligned16(y_even)) return IFX_E_ALIGN;
    if (k != kGeneric || !even_copy_ok(d, dm, nullptr, 0)) return IFX_E_UNSUPPORTED;
    ifx::ConvArgs a = conv_args(d, dm, x_blk, w_blk, bias, mult, shift,
                                (d->flags & IFX_RESIDUAL) ? residual : nullptr, y);
    a.y_even = y_even;
    return hip_status(ifx::launch_conv_split(a, d->kh, d->kw, nullptr, 0, (hipStream_t)stream));
}

int32_t ifx_conv_even_supported(const ifx_conv_desc *d)
{
    Kind k;
    Dims dm;
    if (check_desc(d, &k, &dm) != IFX_OK || k != kGeneric) return 0;
    return even_copy_ok(d, dm, nullptr, 0) ? 1 : 0;
}

ifx_status ifx_conv_kernel_name(const ifx_conv_desc *d, char *buf, size_t len)
{
    Kind k;
    Dims dm;
    ifx_status st = check_desc(d, &k, &dm);
    if (st != IFX_OK) return st;
    if (!buf) return IFX_E_NULL;
    ArmedQuery aq;
    st = run_conv(d, k, dm, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    if (st != IFX_OK) return st;
    return copy_name(aq.q, buf, len);
}

ifx_status ifx_conv_proj_kernel_name(const ifx_conv_desc *d3, const ifx_conv_desc *dp, char *buf, size_t len)
{
    if (!d3 || !dp) return IFX_E_NULL;
    Kind k3, kp;
    Dims m3, mp;
    ifx_status st = check_desc(d3, &k3, &m3);
    if (st != IFX_OK) return st;
    st = check_desc(dp, &kp, &mp);
    if (st != IFX_OK) return st;
    if (k3 != kGeneric || kp != kGeneric || !proj_fusable(d3, dp)) return IFX_E_UNSUPPORTED;
    if (dp->n != d3->n || dp->c_out != d3->c_out || mp.oh != m3.oh || mp.ow != m3.ow) return IFX_E_SHAPE;
    if (!buf) return IFX_E_NULL;
    ArmedQuery aq;
    const ifx::ConvArgs a = conv_args(d3, m3, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    const ifx::ConvArgs pj = conv_args(dp, mp, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    st = hip_status(ifx::launch_conv_proj(a, pj, nullptr));
    if (st != IFX_OK) return st;
    return copy_name(aq.q, buf, len);
}

size_t ifx_block_workspace_bytes(const ifx_block_params *p)
{
    BlockPlan plan;
    if (plan_block(p, 0, &plan) != IFX_OK) return 0;
    return plan.t1 + plan.t2 + plan.sc + plan.part;
}

ifx_status ifx_conv_proj_fused(const ifx_conv_desc *d3, const int8_t *t_blk, const int8_t *w3_blk,
                               const int32_t *bias3, const int32_t *mult3, const int32_t *shift3,
                               const ifx_conv_desc *dp, const int8_t *x_blk, const int8_t *wp_blk,
                               const int32_t *biasp, const int32_t *multp, const int32_t *shiftp,
                               int8_t *y_blk, void *stream)
{
    if (!d3 || !dp) return IFX_E_NULL;
    Kind k3, kp;
    Dims m3, mp;
    ifx_status st = check_desc(d3, &k3, &m3);
    if (st != IFX_OK) return st;
    st = check_desc(dp, &kp, &mp);
    if (st != IFX_OK) return st;
    if (k3 != kGeneric || kp != kGeneric || !proj_fusable(d3, dp)) return IFX_E_UNSUPPORTED;
    if (dp->n != d3->n || dp->c_out != d3->c_out || mp.oh != m3.oh || mp.ow != m3.ow) return IFX_E_SHAPE;
    const void *ptrs[] = {t_blk, w3_blk, bias3, mult3, shift3, x_blk, wp_blk, biasp, multp, shiftp, y_blk};
    for (const void *q : ptrs)
        if (!q) return IFX_E_NULL;
    for (const void *q : ptrs)
        if (!aligned16(q)) return IFX_E_ALIGN;
    const ifx::ConvArgs a = conv_args(d3, m3, t_blk, w3_blk, bias3, mult3, shift3, nullptr, y_blk);
    const ifx::ConvArgs pj = conv_args(dp, mp, x_blk, wp_blk, biasp, multp, shiftp, nullptr, nullptr);
    return hip_status(ifx::launch_conv_proj(a, pj, (hipStream_t)stream));
}

ifx_status ifx_conv_chain_fused(const ifx_conv_desc *d3, const int8_t *t_blk, const int8_t *w3_blk,
                                const int32_t *bias3, const int32_t *mult3, const int32_t *shift3,
                                const int8_t *residual_blk, int8_t *y_blk, const ifx_conv_desc *d1,
                                const int8_t *w1_blk, const int32_t *bias1, const int32_t *mult1,
                                const int32_t *shift1, int8_t *t1_blk, void *stream)
{
    Dims m3, m1;
    ifx_conv_desc d3c;
    bool even;
    ifx_status st = check_chain(d3, d1, &m3, &m1, &d3c, &even);
    if (st != IFX_OK) return st;
    const void *ptrs[] = {t_blk, w3_blk, bias3, mult3, shift3, residual_blk, y_blk, w1_blk, bias1, mult1, shift1, t1_blk};
    for (const void *q : ptrs)
        if (!q) return IFX_E_NULL;
    for (const void *q : ptrs)
        if (!aligned16(q)) return IFX_E_ALIGN;
    ifx::ConvArgs a = conv_args(&d3c, m3, t_blk, w3_blk, bias3, mult3, shift3, residual_blk, y_blk);
    a.out_even = even ? 1 : 0;
    const ifx::ConvArgs b = conv_args(d1, m1, y_blk, w1_blk, bias1, mult1, shift1, nullptr, t1_blk);
    return hip_status(ifx::launch_conv1x1_chain(a, b, (hipStream_t)stream));
}

ifx_status ifx_conv_chain_kernel_name(const ifx_conv_desc *d3, const ifx_conv_desc *d1, char *buf, size_t len)
{
    Dims m3, m1;
    ifx_conv_desc d3c;
    bool even;
    ifx_status st = check_chain(d3, d1, &m3, &m1, &d3c, &even);
    if (st != IFX_OK) return st;
    if (!buf) return IFX_E_NULL;
    ArmedQuery aq;
    ifx::ConvArgs a = conv_args(&d3c, m3, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    a.out_even = even ? 1 : 0;
    const ifx::ConvArgs b = conv_args(d1, m1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    st = hip_status(ifx::launch_conv1x1_chain(a, b, nullptr));
    if (st != IFX_OK) return st;
    return copy_name(aq.q, buf, len);
}

ifx_status ifx_conv_proj_chain_fused(const ifx_conv_desc *d3, const int8_t *t_blk, const int8_t *w3_blk,
                                     const int32_t *bias3, const int32_t *mult3, const int32_t *shift3,
                                     const ifx_conv_desc *dp, const int8_t *x_blk, const int8_t *wp_blk,
                                     const int32_t *biasp, const int32_t *multp, const int32_t *shiftp,
                                     int8_t *y_blk, const ifx_conv_desc *d1, const int8_t *w1_blk,
                                     const int32_t *bias1, const int32_t *mult1, const int32_t *shift1,
                                     int8_t *t1_blk, void *stream)
{
    Dims m3, mp, m1;
    ifx_status st = check_proj_chain(d3, dp, d1, &m3, &mp, &m1);
    if (st != IFX_OK) return st;
    const void *ptrs[] = {t_blk,  w3_blk, bias3, mult3,  shift3, x_blk, wp_blk, biasp,  multp,
                          shiftp, y_blk,  w1_blk, bias1, mult1, shift1, t1_blk};
    for (const void *q : ptrs)
        if (!q) return IFX_E_NULL;
    for (const void *q : ptrs)
        if (!aligned16(q)) return IFX_E_ALIGN;
    const ifx::ConvArgs a = conv_args(d3, m3, t_blk, w3_blk, bias3, mult3, shift3, nullptr, y_blk);
    const ifx::ConvArgs pj = conv_args(dp, mp, x_blk, wp_blk, biasp, multp, shiftp, nullptr, nullptr);
    const ifx::ConvArgs b = conv_args(d1, m1, y_blk, w1_blk, bias1, mult1, shift1, nullptr, t1_blk);
    return hip_status(ifx::launch_conv1x1_proj_chain(a, pj, b, (hipStream_t)stream));
}

ifx_status ifx_conv_proj_chain_kernel_name(const ifx_conv_desc *d3, const ifx_conv_desc *dp,
                                           const ifx_conv_desc *d1, char *buf, size_t len)
{
    Dims m3, mp, m1;
    ifx_status st = check_proj_chain(d3, dp, d1, &m3, &mp, &m1);
    if (st != IFX_OK) return st;
    if (!buf) return IFX_E_NULL;
    ArmedQuery aq;
    const ifx::ConvArgs a = conv_args(d3, m3, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    const ifx::ConvArgs pj = conv_args(dp, mp, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    const ifx::ConvArgs b = conv_args(d1, m1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    st = hip_status(ifx::launch_conv1x1_proj_chain(a, pj, b, nullptr));
    if (st != IFX_OK) return st;
    return copy_name(aq.q, buf, len);
}

ifx_status ifx_block_forward(const ifx_block_params *p, const int8_t *x_blk, int8_t *y_blk, void *ws,
                             size_t ws_bytes, void *stream)
{
    BlockPlan plan;
    ifx_status st = plan_block(p, 0, &plan);
    if (st != IFX_OK) return st;
    st = check_block_ptrs(p);
    if (st != IFX_OK) return st;
    if (!x_blk || !y_blk || !ws) return IFX_E_NULL;
    if (!aligned16(x_blk) || !aligned16(y_blk) || !aligned16(ws)) return IFX_E_ALIGN;
    if (ws_bytes < plan.t1 + plan.t2 + plan.sc + plan.part) return IFX_E_WORKSPACE;
    int32_t *part = (int32_t *)((int8_t *)ws + plan.t1 + plan.t2 + plan.sc);
    return run_block(p, plan, p->d[0].n, x_blk, y_blk, (int8_t *)ws, part, plan.part, (hipStream_t)stream);
}

ifx_status ifx_block_forward_noalloc(const ifx_block_params *p, const int8_t *x_blk, int8_t *y_blk, void *stream)
{
    BlockPlan plan;
    ifx_status st = plan_block(p, 0, &plan);
    if (st != IFX_OK) return st;
    st = check_block_ptrs(p);
    if (st != IFX_OK) return st;
    if (!x_blk || !y_blk) return IFX_E_NULL;
    if (!aligned16(x_blk) || !aligned16(y_blk)) return IFX_E_ALIGN;
    if (plan.t1 + plan.t2 + plan.sc + plan.part > (size_t)IFX_BLOCK_SCRATCH_BYTES) return IFX_E_WORKSPACE;
    int8_t *ws = nullptr;
    st = hip_status(scratch_ptr(&ws));
    if (st != IFX_OK) return st;
    // every byte the kernels read from the scratch (t1, t2, shortcut, split-K partial sums) is
    // written earlier in the same call, so nothing needs clearing
    int32_t *part = (int32_t *)(ws + plan.t1 + plan.t2 + plan.sc);
    return run_block(p, plan, p->d[0].n, x_blk, y_blk, ws, part, plan.part, (hipStream_t)stream);
}

size_t ifx_net_workspace_bytes(const ifx_net_params *p, int32_t n)
{
    NetPlan plan;
    if (plan_net(p, n, &plan) != IFX_OK) return 0;
    return net_ws_bytes(plan);
}

}  // extern "C"

namespace {

// Validation of ifx_net_forward's arguments (nothing is launched).
ifx_status check_net_call(const ifx_net_params *p, const int8_t *x_blk, const int32_t *logits, int32_t n,
                          const void *ws, size_t ws_bytes, NetPlan *plan)
{
    ifx_status st = plan_net(p, n, plan);
    if (st != IFX_OK) return st;
    if (!x_blk || !logits || !ws || !p->stem_w || !p->stem_bias || !p->stem_mult || !p->stem_shift || !p->fc_w_blk ||
        !p->fc_bias)
        return IFX_E_NULL;
    if (!aligned16(x_blk) || !aligned16(logits) || !aligned16(ws) || !aligned16(p->stem_w) ||
        !aligned16(p->stem_bias) || !aligned16(p->stem_mult) || !aligned16(p->stem_shift) ||
        !aligned16(p->fc_w_blk) || !aligned16(p->fc_bias))
        return IFX_E_ALIGN;
    for (int i = 0; i < p->n_blocks; ++i) {
        st = check_block_ptrs(&p->blocks[i]);
        if (st != IFX_OK) return st;
    }
    if (ws_bytes < net_ws_bytes(*plan)) return IFX_E_WORKSPACE;
    return IFX_OK;
}

// The passes of a validated network call.  Pass i runs on lane i % plan.lanes: lane 0 is s0,
// lane 1 is l1's stream, forked from s0 and joined back into it by l1's events.  `lock` (or
// null) is held around the fork and around the join.
ifx_status run_net(const ifx_net_params *p, const NetPlan &plan, const int8_t *x_blk, int32_t *logits, int32_t n,
                   void *ws, hipStream_t s0, const Lane &l1, std::mutex *lock)
{
    const size_t in_img = (p->stem.flags & IFX_INPUT_NHWC)
                              ? (size_t)p->stem.h * p->stem.w * p->stem.c_in
                              : act_bytes(1, p->stem.h, p->stem.w, p->stem.c_in);
    hipStream_t ls[2] = {s0, l1.stream};
    ifx_status st = IFX_OK;
    if (plan.lanes > 1) {
        std::unique_lock<std::mutex> g;
        if (lock) g = std::unique_lock<std::mutex>(*lock);
        st = hip_status(hipEventRecord(l1.fork, s0));
        if (st == IFX_OK) st = hip_status(hipStreamWaitEvent(l1.stream, l1.fork, 0));
        if (st != IFX_OK) return st;
    }
    int pass = 0;
    for (int i0 = 0; i0 < n && st == IFX_OK; i0 += plan.nb, ++pass) {
        const int lane = pass % plan.lanes;
        hipStream_t s = ls[lane];
        int8_t *base = (int8_t *)ws + lane * lane_ws_bytes(plan);
        int8_t *act[2] = {base, base + plan.act};
        int8_t *bws = base + 2 * plan.act;  // t1 | t2 | sc of the current block
        int8_t *pool = bws + plan.t1 + plan.t2 + plan.sc;
        int32_t *part = (int32_t *)(pool + plan.pool);  // split-K partial sums
        const int nb = std::min(plan.nb, n - i0);
        ifx_conv_desc sd = p->stem;
        sd.n = nb;
        Kind k;
        Dims dm;
        st = check_desc(&sd, &k, &dm);
        if (st != IFX_OK) break;
        st = run_conv(&sd, k, dm, x_blk + (size_t)i0 * in_img, p->stem_w, p->stem_bias, p->stem_mult, p->stem_shift,
                      nullptr, act[0], s);
        if (st != IFX_OK) break;
        int cur = 0;
        BlockFlow flow;  // what the previous block left for this one
        for (int b = 0; b < p->n_blocks; ++b) {
            BlockPlan bp;
            st = plan_block(&p->blocks[b], nb, &bp);
            if (st != IFX_OK) break;
            // the block's own workspace pieces are laid out inside the net's t1|t2|sc area
            BlockPlan lay = bp;
            lay.t1 = plan.t1;
            lay.t2 = plan.t2;
            lay.sc = plan.sc;
            const ifx_block_params *next = b + 1 < p->n_blocks ? &p->blocks[b + 1] : nullptr;
            BlockFlow left;
            st = run_block(&p->blocks[b], lay, nb, act[cur], act[cur ^ 1], bws, part, plan.part, s, flow, next,
                           &left);
            if (st != IFX_OK) break;
            flow = left;
            cur ^= 1;
        }
        if (st != IFX_OK) break;
        const int c1 = (plan.out_c + 31) / 32;
        st = hip_status(ifx::launch_avgpool(act[cur], pool, nb, c1, plan.out_h * plan.out_w, s));
        if (st != IFX_OK) break;
        ifx_conv_desc fd = {nb, 1, 1, p->fc_in, p->fc_out, 1, 1, 1, 0, IFX_OUT_I32};
        st = check_desc(&fd, &k, &dm);
        if (st != IFX_OK) break;
        st = run_conv(&fd, k, dm, pool, p->fc_w_blk, p->fc_bias, nullptr, nullptr, nullptr,
                      logits + (size_t)i0 * p->fc_out, s, part, plan.part);
        if (st != IFX_OK) break;
    }
    if (plan.lanes > 1) {
        // the join is enqueued whatever happened above, so s0 always follows every pass
        std::unique_lock<std::mutex> g;
        if (lock) g = std::unique_lock<std::mutex>(*lock);
        ifx_status st2 = hip_status(hipEventRecord(l1.join, l1.stream));
        if (st2 == IFX_OK) st2 = hip_status(hipStreamWaitEvent(s0, l1.join, 0));
        if (st == IFX_OK) st = st2;
    }
    return st;
}

}  // namespace

extern "C" {

ifx_status ifx_net_forward(const ifx_net_params *p, const int8_t *x_blk, int32_t *logits, int32_t n, void *ws,
                           size_t ws_bytes, void *stream)
{
    NetPlan plan;
    ifx_status st = check_net_call(p, x_blk, logits, n, ws, ws_bytes, &plan);
    if (st != IFX_OK) return st;
    hipStream_t s0 = (hipStream_t)stream;
    Lane l1;
    if (plan.lanes > 1) {
        // a stream being captured by the caller keeps every pass on itself: the library's lane
        // is shared by every caller on the device and must not be pulled into a capture
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        st = hip_status(hipStreamIsCapturing(s0, &cap));
        if (st != IFX_OK) return st;
        if (cap != hipStreamCaptureStatusNone) {
            plan.lanes = 1;
        } else {
            std::lock_guard<std::mutex> g(lane_mutex());
            st = hip_status(device_lane(&l1));
            if (st != IFX_OK) return st;
        }
    }
    return run_net(p, plan, x_blk, logits, n, ws, s0, l1, &lane_mutex());
}

// ---------------------------------------------------------------------------
// Fixed-shape network launches recorded once into a HIP graph
// ---------------------------------------------------------------------------
struct ifx_graph_s {
    hipGraph_t graph;
    hipGraphExec_t exec;
};

ifx_status ifx_net_graph_create(const ifx_net_params *p, const int8_t *x_blk, int32_t *logits, int32_t n, void *ws,
                                size_t ws_bytes, ifx_graph *out)
{
    if (!out) return IFX_E_NULL;
    *out = nullptr;
    // validate every argument first: an invalid call records nothing
    NetPlan plan;
    ifx_status st = check_net_call(p, x_blk, logits, n, ws, ws_bytes, &plan);
    if (st != IFX_OK) return st;
    // the recording uses streams and events of its own, created outside the capture and
    // destroyed after it: the recorded graph shares nothing with other callers' work
    hipStream_t cs = nullptr;
    Lane l1;
    st = hip_status(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));  // default priority
    if (st == IFX_OK && plan.lanes > 1) st = hip_status(make_lane(&l1));
    if (st == IFX_OK) st = hip_status(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal));
    if (st != IFX_OK) {
        free_lane(&l1);
        if (cs) (void)hipStreamDestroy(cs);
        return st;
    }
    const ifx_status fst = run_net(p, plan, x_blk, logits, n, ws, cs, l1, nullptr);
    hipGraph_t graph = nullptr;
    st = hip_status(hipStreamEndCapture(cs, &graph));
    free_lane(&l1);
    (void)hipStreamDestroy(cs);
    if (fst != IFX_OK || st != IFX_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return fst != IFX_OK ? fst : st;
    }
    hipGraphExec_t exec = nullptr;
    st = hip_status(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0));
    if (st != IFX_OK) {
        (void)hipGraphDestroy(graph);
        return st;
    }
    *out = new ifx_graph_s{graph, exec};
    return IFX_OK;
}

ifx_status ifx_graph_launch(ifx_graph g, void *stream)
{
    if (!g) return IFX_E_NULL;
    return hip_status(hipGraphLaunch(g->exec, (hipStream_t)stream));
}

ifx_status ifx_graph_destroy(ifx_graph g)
{
    if (!g) return IFX_OK;
    ifx_status st = hip_status(hipGraphExecDestroy(g->exec));
    const ifx_status st2 = hip_status(hipGraphDestroy(g->graph));
    delete g;
    return st != IFX_OK ? st : st2;
}

const char *ifx_status_string(ifx_status s)
{
    switch (s) {
    case IFX_OK: return "ok";
    case IFX_E_NULL: return "null pointer";
    case IFX_E_SHAPE: return "invalid or inconsistent shape";
    case IFX_E_UNSUPPORTED: return "unsupported kernel/stride/pad/flags";
    case IFX_E_ALIGN: return "pointer not 16-byte aligned";
    case IFX_E_WORKSPACE: return "workspace too small";
    case IFX_E_HIP: return "HIP launch failure";
    }
    return "unknown status";
}

int32_t ifx_last_hip_error(void) { return g_last_hip; }

int32_t ifx_version(void) { return 100; }

}  // extern "C"
