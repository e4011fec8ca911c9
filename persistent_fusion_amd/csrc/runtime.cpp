// Host runtime of the persistent small-op queue: contexts, validation, hazard
// dependencies, the fusion pass, ring publication (the doorbell), completion
// tracking, and the per-op launch comparator.
//
// The queue is the "host-managed work queue" of "GPUOS: A GPU Operating
// System Primitive for Transparent Operation Fusion" (section "The Paper"),
// fed in "unified submissions" (one flush publishes many ops).  The hand-off
// follows "Kernel Launch and Host-Device Interaction" (section "The launch
// path"): descriptors go into a pinned ring in host memory and a single store
// of the ring tail acts as the doorbell; the GPU side polls it.  Pinned memory
// is what lets the device read the ring directly (same page, section "Memory
// transfers").
#include <hip/hip_runtime.h>
#include <hip/hiprtc.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <unordered_map>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/gpuos.h"
#include "../../include/gpuos_debug.h"
#include "gpuos_internal.h"
#include "kernels.h"

using namespace gpuos;

namespace gpuos {
// Sources of the compiled kernel variant, embedded at build time under the
// names their #include lines use (rtc_sources.cpp, generated).
extern const char* const kRtcSourceNames[];
extern const char* const kRtcSourceTexts[];
extern const unsigned kRtcSourceCount;
}  // namespace gpuos

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  if (getenv("GPUOS_LOG")) fprintf(stderr, "gpuos: %s\n", buf);
  return code;
}

#define HIP_TRY(expr)                                                              \
  do {                                                                             \
    hipError_t e_ = (expr);                                                        \
    if (e_ != hipSuccess)                                                          \
      return fail(GPUOS_EDEVICE, "%s failed: %s", #expr, hipGetErrorString(e_));   \
  } while (0)

inline uint64_t load_acq(const uint64_t* p) {
  return __atomic_load_n(p, __ATOMIC_ACQUIRE);
}
inline void store_rel(uint64_t* p, uint64_t v) { __atomic_store_n(p, v, __ATOMIC_RELEASE); }

inline void cpu_relax() {
#if defined(__x86_64__)
  __builtin_ia32_pause();
#endif
}

uint32_t elem_size(uint32_t dt) { return dt == GPUOS_BF16 || dt == GPUOS_F16 ? 2u : 4u; }

bool is_elementwise(uint32_t op) {
  switch (op) {
    case GPUOS_OP_COPY: case GPUOS_OP_GATHER: case GPUOS_OP_ADD: case GPUOS_OP_MUL:
    case GPUOS_OP_SCALE: case GPUOS_OP_RELU: case GPUOS_OP_EXP: case GPUOS_OP_SILU_MUL:
      return true;
    default:
      return false;
  }
}

bool is_binary(uint32_t op) {
  return op == GPUOS_OP_ADD || op == GPUOS_OP_MUL || op == GPUOS_OP_SILU_MUL;
}

// ---------------------------------------------------------------------------
// byte ranges an op reads and writes (used by validation and hazards)

struct Range {
  uint64_t lo, hi;
};

// A vector with N elements of inline storage (no heap allocation until it
// holds more than N).
template <class T, unsigned N>
class SmallVec {
 public:
  T* begin() { return n_ <= N ? inl_ : ext_.data(); }
  T* end() { return begin() + n_; }
  const T* begin() const { return n_ <= N ? inl_ : ext_.data(); }
  const T* end() const { return begin() + n_; }
  size_t size() const { return n_; }
  bool empty() const { return n_ == 0; }
  T& operator[](size_t i) { return begin()[i]; }
  const T& operator[](size_t i) const { return begin()[i]; }
  T& back() { return begin()[n_ - 1]; }
  void clear() {
    n_ = 0;
    ext_.clear();
  }
  void push_back(const T& x) {
    if (n_ < N) {
      inl_[n_++] = x;
      return;
    }
    if (n_ == N) ext_.assign(inl_, inl_ + N);
    ext_.push_back(x);
    ++n_;
  }
  // keeps the first k elements
  void truncate(size_t k) {
    if (k >= n_) return;
    if (n_ > N) {
      if (k <= N) {
        std::copy(ext_.begin(), ext_.begin() + k, inl_);
        ext_.clear();
      } else {
        ext_.resize(k);
      }
    }
    n_ = (uint32_t)k;
  }
  template <class Pred>
  void remove_if(Pred p) {
    truncate((size_t)(std::remove_if(begin(), end(), p) - begin()));
  }
  void sort_unique() {
    if (n_ <= 1) return;
    T* a = begin();
    if (n_ <= 16) {
      for (uint32_t i = 1; i < n_; ++i) {  // insertion sort: lists are short
        const T v = a[i];
        uint32_t j = i;
        for (; j > 0 && v < a[j - 1]; --j) a[j] = a[j - 1];
        a[j] = v;
      }
    } else {
      std::sort(a, a + n_);
    }
    truncate((size_t)(std::unique(a, a + n_) - a));
  }

 private:
  T inl_[N];
  uint32_t n_ = 0;
  std::vector<T> ext_;
};

typedef SmallVec<uint64_t, 8> DepVec;

struct OpRanges {
  Range w{0, 0};
  Range r[3]{};
  int nr = 0;
};

// An elementwise op's view after normalisation (gpuos_view): dimensions of
// extent 1 dropped, adjacent dimensions merged wherever every operand's
// strides allow, then padded to 4 with leading extents of 1.  on = 0: no view.
// A FIFO of 64-bit words with O(1) indexing: one power-of-two array used as
// a ring (the id -> sequence map is indexed on every dependency check, where
// std::deque's two-level lookup showed).
class WordFifo {
 public:
  size_t size() const { return n_; }
  bool empty() const { return n_ == 0; }
  uint64_t& operator[](size_t i) { return a_[(head_ + i) & (a_.size() - 1)]; }
  uint64_t operator[](size_t i) const { return a_[(head_ + i) & (a_.size() - 1)]; }
  uint64_t front() const { return a_[head_]; }
  void pop_front() {
    head_ = (head_ + 1) & (a_.size() - 1);
    --n_;
  }
  void push_back(uint64_t v) {
    if (n_ == a_.size()) grow();
    a_[(head_ + n_) & (a_.size() - 1)] = v;
    ++n_;
  }

 private:
  void grow() {
    std::vector<uint64_t> b(a_.empty() ? 1024 : 2 * a_.size());
    for (size_t i = 0; i < n_; ++i) b[i] = (*this)[i];
    a_.swap(b);
    head_ = 0;
  }
  std::vector<uint64_t> a_;
  size_t head_ = 0, n_ = 0;
};

struct ViewDesc {
  uint32_t on = 0;
  uint32_t shape[4] = {1, 1, 1, 1};
  uint32_t stride[3][4] = {};  // elements: out, in0, in1
  // largest element offset of operand k
  uint64_t max_off(int k) const {
    uint64_t m = 0;
    for (int d = 0; d < 4; ++d) m += (uint64_t)(shape[d] - 1) * stride[k][d];
    return m;
  }
};

// A PROGRAM op's body as its descriptor carries it (dwords 26-50; see the
// pg layout): meta = n_insns | result << 8 | n_inputs << 16 | zero mask << 24,
// where the zero mask lists the per-element registers r0..r7 the program
// reads before writing (they start at +0).
struct ProgCode {
  uint32_t meta = 0;
  uint32_t ins[GPUOS_PROG_MAX_INSNS] = {};
  float k[8] = {};
  uint32_t n_inputs() const { return (meta >> 16) & 3u; }
};
static_assert(sizeof(ProgCode) == 100, "a body's bytes are its identity: no padding");

// Arity of a program instruction: registers it reads.
int pop_arity(uint32_t op) {
  switch (op) {
    case GPUOS_P_ADD: case GPUOS_P_SUB: case GPUOS_P_MUL: case GPUOS_P_DIV:
    case GPUOS_P_MIN: case GPUOS_P_MAX: case GPUOS_P_LT:
      return 2;
    case GPUOS_P_SEL:
      return 3;
    default:
      return 1;
  }
}

int check_program(const gpuos_program* p, ProgCode& out) {
  if (!p) return fail(GPUOS_EINVAL, "program is null");
  if (p->n_insns < 1 || p->n_insns > GPUOS_PROG_MAX_INSNS)
    return fail(GPUOS_EINVAL, "program: n_insns %u outside 1..%d", p->n_insns, GPUOS_PROG_MAX_INSNS);
  if (p->n_inputs < 1 || p->n_inputs > 3) return fail(GPUOS_EINVAL, "program: n_inputs %u outside 1..3", p->n_inputs);
  if (p->result > 15) return fail(GPUOS_EINVAL, "program: result register %u > 15", p->result);
  if (p->_reserved) return fail(GPUOS_EINVAL, "program: reserved field is not 0");
  out = ProgCode{};
  uint32_t written = (1u << p->n_inputs) - 1, zmask = 0;
  auto reads = [&](uint32_t r) {
    if (r < 8 && !(written & (1u << r))) zmask |= 1u << r;
  };
  for (uint32_t s = 0; s < p->n_insns; ++s) {
    const gpuos_insn& in = p->insns[s];
    if (in.op >= GPUOS_P_COUNT) return fail(GPUOS_EINVAL, "program: instruction %u: unknown op %u", s, in.op);
    if (in.dst > 7) return fail(GPUOS_EINVAL, "program: instruction %u: destination r%u is not 0..7", s, in.dst);
    const int ar = pop_arity(in.op);
    const uint8_t src[3] = {in.a, in.b, in.c};
    for (int j = 0; j < 3; ++j) {
      if (j < ar && src[j] > 15)
        return fail(GPUOS_EINVAL, "program: instruction %u: source register %u > 15", s, src[j]);
      if (j >= ar && src[j])
        return fail(GPUOS_EINVAL, "program: instruction %u: unused operand field is not 0", s);
    }
    if (in._reserved[0] || in._reserved[1] || in._reserved[2])
      return fail(GPUOS_EINVAL, "program: instruction %u: reserved field is not 0", s);
    for (int j = 0; j < ar; ++j) reads(src[j]);
    written |= 1u << in.dst;
    out.ins[s] = in.op | (uint32_t)in.dst << 5 | (uint32_t)in.a << 8 | (uint32_t)in.b << 12 |
                 (uint32_t)in.c << 16;
  }
  for (uint32_t s = p->n_insns; s < GPUOS_PROG_MAX_INSNS; ++s) {
    const gpuos_insn& in = p->insns[s];
    if (in.op || in.dst || in.a || in.b || in.c || in._reserved[0] || in._reserved[1] || in._reserved[2])
      return fail(GPUOS_EINVAL, "program: instruction slot %u past n_insns is not 0", s);
  }
  reads(p->result);
  for (int j = 0; j < 8; ++j) out.k[j] = p->consts[j];
  out.meta = p->n_insns | p->result << 8 | p->n_inputs << 16 | zmask << 24;
  return 0;
}

uint64_t src_extent(uint64_t src_len, uint64_t extent) {
  if (src_len == 0 || src_len >= extent) return extent;
  return src_len;
}

OpRanges op_ranges(const gpuos_op& o, const ViewDesc* v = nullptr) {
  OpRanges R;
  const uint64_t es = elem_size(o.dtype);
  auto rd = [&](const void* p, uint64_t bytes) {
    if (p && bytes) R.r[R.nr++] = Range{(uint64_t)p, (uint64_t)p + bytes};
  };
  auto wr = [&](void* p, uint64_t bytes) {
    if (p && bytes) R.w = Range{(uint64_t)p, (uint64_t)p + bytes};
  };
  const uint64_t n = o.n;
  if (v && v->on) {  // each operand from its pointer to its largest offset
    wr(o.out, (v->max_off(0) + 1) * es);
    rd(o.in[0], (v->max_off(1) + 1) * es);
    if (is_binary(o.opcode)) rd(o.in[1], (v->max_off(2) + 1) * es);
    return R;
  }
  switch (o.opcode) {
    case GPUOS_OP_COPY: case GPUOS_OP_ADD: case GPUOS_OP_MUL: case GPUOS_OP_SCALE:
    case GPUOS_OP_RELU: case GPUOS_OP_EXP: case GPUOS_OP_SILU_MUL:
      wr(o.out, n * es);
      rd(o.in[0], src_extent(o.src_len[0], n) * es);
      if (is_binary(o.opcode)) rd(o.in[1], src_extent(o.src_len[1], n) * es);
      break;
    case GPUOS_OP_GATHER:
      wr(o.out, n * es);
      rd(o.in[0], o.src_len[0] * es);
      rd(o.in[2], n * 4);
      break;
    case GPUOS_OP_PROGRAM:  // data inputs in[0..n_inputs)
      wr(o.out, n * es);
      for (int j = 0; j < 3; ++j) rd(o.in[j], n * es);
      break;
    case GPUOS_OP_ROW_SUM:
      wr(o.out, (uint64_t)o.rows * es);
      rd(o.in[0], src_extent(o.src_len[0], n) * es);
      break;
    case GPUOS_OP_ROW_SOFTMAX:
      wr(o.out, n * es);
      rd(o.in[0], src_extent(o.src_len[0], n) * es);
      break;
    case GPUOS_OP_RMSNORM:
      wr(o.out, n * es);
      rd(o.in[0], src_extent(o.src_len[0], n) * es);
      rd(o.in[2], (uint64_t)o.row_len * es);
      break;
    case GPUOS_OP_ROPE:
      wr(o.out, n * es);
      rd(o.in[0], n * es);
      rd(o.in[2], (uint64_t)o.row_len * 4);
      break;
    case GPUOS_OP_GEMV:
      wr(o.out, (uint64_t)o.aux[0] * es);
      rd(o.in[0], (uint64_t)o.aux[1] * es);
      rd(o.in[2], (uint64_t)o.aux[0] * (uint64_t)o.aux[1] * 2);
      break;
    case GPUOS_OP_ATTN_SCORE: {
      const uint64_t H = o.aux[0], D = o.aux[1], S = o.aux[2];
      wr(o.out, H * S * 4);
      rd(o.in[0], H * D * es);
      rd(o.in[2], S * H * D * 2);
      break;
    }
    case GPUOS_OP_ATTN_AV: {
      const uint64_t H = o.aux[0], D = o.aux[1], S = o.aux[2];
      wr(o.out, H * D * es);
      rd(o.in[0], H * S * 4);
      rd(o.in[2], S * H * D * 2);
      break;
    }
    default:
      break;
  }
  return R;
}

bool overlaps(const Range& a, const Range& b) {
  return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo;
}

// ---------------------------------------------------------------------------
// validation

int validate(const gpuos_op& o, uint32_t index, bool has_view = false) {
  const uint32_t op = o.opcode;
  if (op >= GPUOS_OP_COUNT) return fail(GPUOS_EINVAL, "op %u: unknown opcode %u", index, op);
  if (o.dtype > GPUOS_F16) return fail(GPUOS_EINVAL, "op %u: unknown dtype %u", index, o.dtype);
  if (o.flags & ~0x7u) return fail(GPUOS_EINVAL, "op %u: unknown flag bits 0x%x", index, o.flags);
  if (o.dtype == GPUOS_I32 && op != GPUOS_OP_COPY && op != GPUOS_OP_GATHER && op != GPUOS_OP_ADD &&
      op != GPUOS_OP_MUL && op != GPUOS_OP_RELU)
    return fail(GPUOS_EINVAL, "op %u: int32 is only for COPY, GATHER, ADD, MUL and RELU", index);
  if (o.dtype == GPUOS_F16 &&
      (op == GPUOS_OP_GATHER || op == GPUOS_OP_GEMV || op == GPUOS_OP_ATTN_SCORE || op == GPUOS_OP_ATTN_AV))
    return fail(GPUOS_EINVAL, "op %u: fp16 is not available for this opcode", index);
  const uint64_t es = elem_size(o.dtype);
  auto need = [&](const void* p, const char* what) -> int {
    if (!p) return fail(GPUOS_EINVAL, "op %u: %s pointer is null", index, what);
    return 0;
  };
  auto align = [&](const void* p, uint64_t a, const char* what) -> int {
    if (p && ((uintptr_t)p % a)) return fail(GPUOS_EINVAL, "op %u: %s not %llu-byte aligned",
                                             index, what, (unsigned long long)a);
    return 0;
  };
  int rc;
  if (op == GPUOS_OP_NOP) return 0;
  if (op == GPUOS_OP_SPIN) {
    if (o.aux[0] < 0) return fail(GPUOS_EINVAL, "op %u: negative spin time", index);
    return 0;
  }
  if (o.n == 0) return fail(GPUOS_EINVAL, "op %u: n must be > 0", index);
  if ((rc = need(o.out, "out"))) return rc;
  if ((rc = need(o.in[0], "in[0]"))) return rc;
  if ((rc = align(o.out, es, "out"))) return rc;
  if ((rc = align(o.in[0], es, "in[0]"))) return rc;
  if (o.src_len[0] > (1ull << 30) || o.src_len[1] > (1ull << 30) || o.n > (1u << 30))
    return fail(GPUOS_EINVAL, "op %u: n and src_len are limited to 2^30 elements", index);
  if (is_binary(op)) {
    if ((rc = need(o.in[1], "in[1]"))) return rc;
    if ((rc = align(o.in[1], es, "in[1]"))) return rc;
  }
  switch (op) {
    case GPUOS_OP_GATHER:
      if ((rc = need(o.in[2], "index"))) return rc;
      if ((rc = align(o.in[2], 4, "index"))) return rc;
      if (o.src_len[0] == 0) return fail(GPUOS_EINVAL, "op %u: GATHER needs src_len[0]", index);
      break;
    case GPUOS_OP_ROW_SUM: case GPUOS_OP_ROW_SOFTMAX: case GPUOS_OP_RMSNORM:
      if (o.rows == 0 || o.row_len == 0 || (uint64_t)o.rows * o.row_len != o.n)
        return fail(GPUOS_EINVAL, "op %u: row op needs n == rows * row_len", index);
      if (o.row_len > 4096) return fail(GPUOS_EINVAL, "op %u: row_len > 4096", index);
      if (op == GPUOS_OP_RMSNORM) {
        if ((rc = need(o.in[2], "gain"))) return rc;
        if ((rc = align(o.in[2], es, "gain"))) return rc;
        if (!(o.eps >= 0.0f)) return fail(GPUOS_EINVAL, "op %u: eps must be >= 0", index);
      }
      break;
    case GPUOS_OP_PROGRAM:
      if (o.src_len[0] || o.src_len[1]) return fail(GPUOS_EINVAL, "op %u: a PROGRAM op takes no src_len", index);
      if (o.aux[0] < 0) return fail(GPUOS_EINVAL, "op %u: negative program id", index);
      if ((rc = align(o.in[1], es, "in[1]")) || (rc = align(o.in[2], es, "in[2]"))) return rc;
      break;
    case GPUOS_OP_ROPE:
      if (o.rows == 0 || o.row_len == 0 || (o.row_len & 1) ||
          (uint64_t)o.rows * o.row_len != o.n)
        return fail(GPUOS_EINVAL, "op %u: ROPE needs n == heads * head_dim, even head_dim", index);
      if ((rc = need(o.in[2], "table"))) return rc;
      if ((rc = align(o.in[2], 4, "table"))) return rc;
      break;
    case GPUOS_OP_GEMV:
      if (o.aux[0] <= 0 || o.aux[1] <= 0 || (uint32_t)o.aux[0] != o.n)
        return fail(GPUOS_EINVAL, "op %u: GEMV needs aux = {M, K} with n == M", index);
      if ((rc = need(o.in[2], "weight"))) return rc;
      if ((rc = align(o.in[2], 2, "weight"))) return rc;
      break;
    case GPUOS_OP_ATTN_SCORE: case GPUOS_OP_ATTN_AV: {
      if (o.aux[0] <= 0 || o.aux[1] <= 0 || o.aux[2] <= 0)
        return fail(GPUOS_EINVAL, "op %u: attention needs aux = {H, D, S}", index);
      const uint64_t H = o.aux[0], D = o.aux[1], S = o.aux[2];
      if (op == GPUOS_OP_ATTN_SCORE && H * S != o.n)
        return fail(GPUOS_EINVAL, "op %u: ATTN_SCORE needs n == H * S", index);
      if (op == GPUOS_OP_ATTN_AV && H * D != o.n)
        return fail(GPUOS_EINVAL, "op %u: ATTN_AV needs n == H * D", index);
      if ((rc = need(o.in[2], "cache"))) return rc;
      if ((rc = align(o.in[2], 2, "cache"))) return rc;
      if (op == GPUOS_OP_ATTN_AV && ((uintptr_t)o.in[0] % 4))
        return fail(GPUOS_EINVAL, "op %u: probabilities must be fp32 aligned", index);
      break;
    }
    default:
      break;
  }
  // the kernels address every operand with 32-bit byte offsets
  const OpRanges R = op_ranges(o);
  if (R.w.hi - R.w.lo > kMaxExtentBytes)
    return fail(GPUOS_EINVAL, "op %u: output spans more than 4 GiB - 1 MiB", index);
  for (int q = 0; q < R.nr; ++q)
    if (R.r[q].hi - R.r[q].lo > kMaxExtentBytes)
      return fail(GPUOS_EINVAL, "op %u: an operand spans more than 4 GiB - 1 MiB", index);
  // In place: tiles run concurrently, so an output may overlap only a data
  // input that is exactly it, read element for element (no cyclic reuse),
  // and only in opcodes whose tiles read an element just where they write it.
  // (A view's overlap rule is checked with the view.)
  if (!has_view) {
    const bool same_index = (is_elementwise(op) && op != GPUOS_OP_GATHER) || op == GPUOS_OP_ROW_SOFTMAX ||
                            op == GPUOS_OP_RMSNORM || op == GPUOS_OP_ROPE || op == GPUOS_OP_PROGRAM;
    // data inputs come first in op_ranges: in[0], then in[1] for binary ops
    // (every read of a PROGRAM op is a data input)
    const int n_data = op == GPUOS_OP_PROGRAM ? R.nr : is_elementwise(op) && is_binary(op) ? 2 : 1;
    for (int q = 0; q < R.nr; ++q) {
      if (!overlaps(R.w, R.r[q])) continue;
      const bool exact = R.r[q].lo == R.w.lo && R.r[q].hi == R.w.hi;
      if (!(same_index && q < n_data && exact))
        return fail(GPUOS_EINVAL, "op %u: the output overlaps an input without being that input "
                    "read element for element", index);
    }
  }
  return 0;
}

// Checks op `index`'s view and normalises it into `out` (out.on = 0 when the
// view is plain contiguous indexing); see gpuos_view.
int normalize_view(const gpuos_op& o, const gpuos_view& v, uint32_t index, ViewDesc& out) {
  out = ViewDesc{};
  if (v.ndim == 0) return 0;
  const uint32_t op = o.opcode;
  if (!is_elementwise(op) || op == GPUOS_OP_GATHER)
    return fail(GPUOS_EINVAL, "op %u: views are only for COPY, ADD, MUL, SCALE, RELU, EXP, SILU_MUL", index);
  if (v.ndim > 4 || v._reserved) return fail(GPUOS_EINVAL, "op %u: malformed view", index);
  if (o.src_len[0] || o.src_len[1]) return fail(GPUOS_EINVAL, "op %u: an op with a view takes no src_len", index);
  const bool bin = is_binary(op);
  const int nk = bin ? 3 : 2;
  struct Dim {
    uint64_t ext;
    int64_t st[3];
  };
  Dim dims[4];
  int nd = 0;
  uint64_t prod = 1;
  for (uint32_t d = 0; d < v.ndim; ++d) {
    const uint64_t ext = v.shape[d];
    if (ext == 0 || ext > (1ull << 30)) return fail(GPUOS_EINVAL, "op %u: view extent %llu", index, (unsigned long long)ext);
    prod *= ext;
    if (prod > (1ull << 30)) return fail(GPUOS_EINVAL, "op %u: view extents exceed 2^30 elements", index);
    for (int k = 0; k < nk; ++k)
      if (v.stride[k][d] < 0 || v.stride[k][d] > 0x7fffffff)
        return fail(GPUOS_EINVAL, "op %u: view stride out of range", index);
    if (ext > 1) dims[nd++] = Dim{ext, {v.stride[0][d], v.stride[1][d], bin ? v.stride[2][d] : 0}};
  }
  if (prod != o.n)
    return fail(GPUOS_EINVAL, "op %u: view extents multiply to %llu, not n = %u", index, (unsigned long long)prod, o.n);
  // merge a dimension into the next inner one wherever every operand steps
  // over the inner one contiguously
  Dim m[4];
  int nm = 0;
  for (int d = nd - 1; d >= 0; --d) {
    if (nm > 0) {
      Dim& in = m[nm - 1];
      bool ok = true;
      for (int k = 0; k < 3; ++k) ok = ok && dims[d].st[k] == in.st[k] * (int64_t)in.ext;
      if (ok) {
        in.ext *= dims[d].ext;
        continue;
      }
    }
    m[nm++] = dims[d];  // m is innermost first
  }
  const uint64_t es = elem_size(o.dtype);
  uint64_t maxoff[3] = {0, 0, 0};
  for (int k = 0; k < nk; ++k) {
    for (int i = 0; i < nm; ++i) maxoff[k] += (m[i].ext - 1) * (uint64_t)m[i].st[k];
    if ((maxoff[k] + 1) * es > kMaxExtentBytes)
      return fail(GPUOS_EINVAL, "op %u: a view operand spans more than 4 GiB - 1 MiB", index);
  }
  // the output must address each element once: ordered by stride, every
  // stride must exceed the span of the smaller ones
  {
    int order[4];
    for (int i = 0; i < nm; ++i) order[i] = i;
    std::sort(order, order + nm, [&](int x, int y) { return m[x].st[0] < m[y].st[0]; });
    uint64_t span = 0;
    for (int i = 0; i < nm; ++i) {
      const Dim& dm = m[order[i]];
      if (dm.st[0] == 0 || (uint64_t)dm.st[0] <= span)
        return fail(GPUOS_EINVAL, "op %u: the view's output addresses an element twice", index);
      span += (dm.ext - 1) * (uint64_t)dm.st[0];
    }
  }
  // an output overlapping an input must be that input under the same view
  const Range ro{(uint64_t)o.out, (uint64_t)o.out + (maxoff[0] + 1) * es};
  for (int k = 1; k < nk; ++k) {
    const Range rk{(uint64_t)o.in[k - 1], (uint64_t)o.in[k - 1] + (maxoff[k] + 1) * es};
    if (!overlaps(ro, rk)) continue;
    bool same = o.in[k - 1] == o.out;
    for (int i = 0; i < nm && same; ++i) same = m[i].st[k] == m[i].st[0];
    if (!same) return fail(GPUOS_EINVAL, "op %u: the output overlaps input %d under a different view", index, k - 1);
  }
  bool plain = nm <= 1;
  for (int i = 0; i < nm && plain; ++i)
    for (int k = 0; k < nk; ++k) plain = plain && m[i].st[k] == 1;
  if (plain) return 0;  // contiguous after all
  out.on = 1;
  for (int i = 0; i < nm; ++i) {  // innermost is dimension 3
    out.shape[3 - i] = (uint32_t)m[i].ext;
    for (int k = 0; k < 3; ++k) out.stride[k][3 - i] = (uint32_t)m[i].st[k];
  }
  return 0;
}

// ---------------------------------------------------------------------------
// hazard map.  Writes keep exact non-overlapping byte segments, each with its
// last writer (user op id) and the readers of that write.  A read never splits
// a segment: it is recorded as a reader of every segment it touches, which can
// only add write-after-read orderings.  Reads of bytes no queued op has
// written (inputs uploaded before the queue) go to merged read spans, so
// reading many different prefixes of one buffer costs no segments.  A write
// depends on the writers and readers of every segment and span it overlaps.
// An index from each segment's first byte to the segment serves the common
// accesses, which start exactly at a segment (reading or rewriting a whole
// earlier output), without a search of the ordered map.

typedef SmallVec<uint64_t, 4> Readers;

struct WSeg {
  uint64_t hi;
  uint64_t writer;
  Readers readers;
};

struct RSpan {
  uint64_t hi;
  Readers readers;
};

class HazardMap {
 public:
  template <class Retired>
  void access(const Range& rg, uint64_t id, bool write, DepVec& deps, Retired retired) {
    if (rg.hi <= rg.lo) return;
    if (write)
      do_write(rg, id, deps, retired);
    else
      do_read(rg, id, deps, retired);
  }

  template <class Retired>
  void prune(Retired retired) {
    for (auto it = w_.begin(); it != w_.end();) {
      WSeg& sg = it->second;
      if (sg.writer && retired(sg.writer)) sg.writer = 0;
      sg.readers.remove_if(retired);
      if (!sg.writer && sg.readers.empty()) {
        wi_.erase(it->first);
        it = w_.erase(it);
      } else {
        ++it;
      }
    }
    for (auto it = r_.begin(); it != r_.end();) {
      it->second.readers.remove_if(retired);
      if (it->second.readers.empty())
        it = r_.erase(it);
      else
        ++it;
    }
  }

  size_t size() const { return w_.size() + r_.size(); }
  void clear() {
    w_.clear();
    wi_.clear();
    r_.clear();
  }

 private:
  // first element whose range may overlap [lo, ...)
  template <class M>
  static typename M::iterator first_overlap(M& m, uint64_t lo) {
    auto it = m.upper_bound(lo);
    if (it != m.begin()) {
      auto p = std::prev(it);
      if (p->second.hi > lo) return p;
    }
    return it;
  }

  template <class Retired>
  static void add_reader(Readers& rd, uint64_t id, Retired retired) {
    if (!rd.empty() && rd.back() == id) return;
    rd.push_back(id);
    const size_t n = rd.size();
    if (n >= 32 && (n & (n - 1)) == 0) rd.remove_if(retired);  // amortised
  }

  template <class Retired>
  void do_read(const Range& rg, uint64_t id, DepVec& deps, Retired retired) {
    const auto f = wi_.find(rg.lo);
    if (f != wi_.end() && f->second->second.hi >= rg.hi) {  // inside one segment
      WSeg& sg = f->second->second;
      if (sg.writer && !retired(sg.writer)) deps.push_back(sg.writer);
      add_reader(sg.readers, id, retired);
      return;
    }
    uint64_t cur = rg.lo;
    bool gap = false;
    for (auto it = first_overlap(w_, rg.lo); it != w_.end() && it->first < rg.hi; ++it) {
      if (it->first > cur) gap = true;
      WSeg& sg = it->second;
      if (sg.writer && !retired(sg.writer)) deps.push_back(sg.writer);
      add_reader(sg.readers, id, retired);
      cur = sg.hi;
    }
    if (gap || cur < rg.hi) add_span(rg, id, retired);
  }

  // records a read of never-written bytes (conservatively the whole range)
  template <class Retired>
  void add_span(const Range& rg, uint64_t id, Retired retired) {
    auto it = first_overlap(r_, rg.lo);
    if (it != r_.end() && it->first <= rg.lo && it->second.hi >= rg.hi) {
      add_reader(it->second.readers, id, retired);  // inside one span
      return;
    }
    // merge every span that overlaps or touches the range into one
    uint64_t lo = rg.lo, hi = rg.hi;
    Readers rd;
    auto j = r_.upper_bound(lo);
    if (j != r_.begin() && std::prev(j)->second.hi >= lo) --j;
    while (j != r_.end() && j->first <= hi) {
      lo = std::min(lo, j->first);
      hi = std::max(hi, j->second.hi);
      for (uint64_t x : j->second.readers) rd.push_back(x);
      j = r_.erase(j);
    }
    rd.remove_if(retired);
    rd.sort_unique();
    add_reader(rd, id, retired);
    r_.emplace(lo, RSpan{hi, std::move(rd)});
  }

  template <class Retired>
  void do_write(const Range& rg, uint64_t id, DepVec& deps, Retired retired) {
    // read spans: every reader of an overlapping span must read first
    for (auto it = first_overlap(r_, rg.lo); it != r_.end() && it->first < rg.hi;) {
      for (uint64_t x : it->second.readers)
        if (!retired(x)) deps.push_back(x);
      if (it->first >= rg.lo && it->second.hi <= rg.hi)
        it = r_.erase(it);  // wholly overwritten
      else
        ++it;
    }
    const auto f = wi_.find(rg.lo);
    if (f != wi_.end() && f->second->second.hi == rg.hi) {
      // exactly one segment (segments never overlap)
      WSeg& sg = f->second->second;
      collect(sg, deps, retired);
      sg.writer = id;
      sg.readers.clear();
      return;
    }
    for (auto j = first_overlap(w_, rg.lo); j != w_.end() && j->first < rg.hi; ++j)
      collect(j->second, deps, retired);
    split(rg.lo);
    split(rg.hi);
    for (auto j = w_.lower_bound(rg.lo); j != w_.end() && j->first < rg.hi;) {
      wi_.erase(j->first);
      j = w_.erase(j);
    }
    wi_[rg.lo] = w_.emplace(rg.lo, WSeg{rg.hi, id, {}}).first;
  }

  template <class Retired>
  static void collect(const WSeg& sg, DepVec& deps, Retired retired) {
    if (sg.writer && !retired(sg.writer)) deps.push_back(sg.writer);
    for (uint64_t r : sg.readers)
      if (!retired(r)) deps.push_back(r);
  }

  void split(uint64_t x) {
    auto it = w_.upper_bound(x);
    if (it == w_.begin()) return;
    --it;
    if (it->first < x && x < it->second.hi) {
      WSeg tail = it->second;
      it->second.hi = x;
      wi_[x] = w_.emplace(x, std::move(tail)).first;
    }
  }

  std::map<uint64_t, WSeg> w_;
  std::unordered_map<uint64_t, std::map<uint64_t, WSeg>::iterator> wi_;  // first byte -> segment
  std::map<uint64_t, RSpan> r_;
};

}  // namespace

// ---------------------------------------------------------------------------
// context

// A loaded compiled kernel variant (gpuos_program_compile): its module, the
// kernel, and the index of each compiled body by the body's bytes.
struct RtcModule {
  hipModule_t mod = nullptr;
  hipFunction_t fn = nullptr;
  std::map<std::string, uint32_t> index;
  uint32_t dtypes = 0;
  bool leak = false;  // a launch of it may still run: never unloaded
  ~RtcModule() {
    if (mod && !leak) (void)hipModuleUnload(mod);
  }
};

std::string body_key(const ProgCode& pc) {
  return std::string(reinterpret_cast<const char*>(&pc), sizeof pc);
}

struct Staged {
  gpuos_op op;
  uint64_t id;
  uint32_t ring;
  DepVec deps;  // user ids
  ViewDesc view;
  ProgCode prog;  // PROGRAM ops: the body as of submission
};

// A device op after the fusion pass: one descriptor built from user ops
// [first, first + count) of the staged list.
struct Planned {
  size_t first;
  uint32_t count;
  DevDesc desc;
  DepVec deps;  // user ids outside the group
  uint32_t ring;
};

struct gpuos_ctx {
  int device = GPUOS_DEVICE_NONE;
  bool host_only = true;
  gpuos_config cfg{};
  hipStream_t stream = nullptr;
  uint32_t cap = 0, cus = 0, blocks = 0, workers = 0, lc_waves = 0;

  // pinned host memory (malloc'd in host-only mode)
  HostCtl* hctl = nullptr;
  DevDesc* hdesc[kRings] = {nullptr, nullptr};
  uint64_t* hends[kRings] = {nullptr, nullptr};
  uint64_t* hdone_lc = nullptr;  // latency-critical completions by slot
  // device memory
  DevCtl* dctl = nullptr;
  DevDesc* ddesc[kRings] = {nullptr, nullptr};
  uint64_t* dends[kRings] = {nullptr, nullptr};
  uint64_t* done_id[kRings] = {nullptr, nullptr};
  uint32_t* tiles_done[kRings] = {nullptr, nullptr};
  uint32_t* subs_done[kRings] = {nullptr, nullptr};
  TraceRec* trace[kRings] = {nullptr, nullptr};
  uint32_t* tile_exec[kRings] = {nullptr, nullptr};
  bool spread_big = false;  // per-op launches: big elementwise ops take every
                            // wave (each op is then the only kernel running)
  bool static_mem = false;  // rings in the caller's workspace and the static
                            // device scratch (gpuos_create_static): not freed

  // host bookkeeping
  uint64_t next_id = 1;
  uint64_t id_base = 1;            // ids below are retired and forgotten
  WordFifo idseq;                  // (ring << 63) | seq, 0 = staged
  std::vector<Staged> staged;
  std::vector<Planned> plan;       // fusion pass output, reused across flushes
  std::vector<uint8_t> tail_ok;    // plan[i..] all runnable by the compiled variant
  uint64_t pub_seq[kRings] = {0, 0};
  uint64_t pub_tiles[kRings] = {0, 0};
  uint64_t tail_written[kRings] = {0, 0};
  // per ring slot of descriptor s: a k such that descriptors 1..k of the
  // ring have all completed whenever s starts (publish_one)
  std::vector<uint64_t> done_prefix[kRings];
  HazardMap hazards;
  std::vector<ProgCode> programs;  // gpuos_program_define / _update
  uint64_t since_prune = 0;
  bool poisoned = false;
  bool consumer = false;    // host-only: another thread plays the device
                            // (gpuos_debug_consumer_attach), so waits block
  bool stopped = false;     // STOP published; no more submissions
  bool exited = false;      // resident kernel has exited
  bool parked = false;      // the kernel left at gpuos_yield; the next flush
  uint64_t park_tiles = 0;  // with work relaunches it from this ticket
  bool leaked = false;      // kernel did not exit: memory must not be freed
  bool timing = false;      // ev_start/ev_end bracket a launch not yet counted
  uint32_t epoch = 0;       // launches so far
  // compiled kernel variants: the latest compile, and the one the running
  // kernel was launched from (null while the built-in kernel runs).  A
  // variant is unloaded once neither holds it.
  std::shared_ptr<RtcModule> rtc_new, rtc_run;
  bool on_rtc = false;      // the launched kernel is rtc_run's
  std::string arch = "gfx950";  // the device's target name for hipRTC
  std::string rtc_source;   // body source of the last compile
  KArgs kargs{};
  hipEvent_t ev_start = nullptr, ev_end = nullptr;
  gpuos_stats st{};
};

namespace {

uint64_t completed_of(gpuos_ctx* c, uint32_t ring) { return load_acq(&c->hctl->completed[ring]); }

bool check_device_error(gpuos_ctx* c) {
  if (c->poisoned) return true;
  const uint64_t e = load_acq(&c->hctl->error);
  if (e) {
    c->poisoned = true;
    c->st.device_error = e;
    c->st.error_desc = c->hctl->error_seq;
    fail(GPUOS_EDEVICE, "device error %llu at ring %llu seq %llu", (unsigned long long)e,
         (unsigned long long)(c->hctl->error_seq >> 62),
         (unsigned long long)(c->hctl->error_seq & ((1ull << 62) - 1)));
    return true;
  }
  return false;
}

// Is user op `id` known to have completed?
bool id_retired(gpuos_ctx* c, uint64_t id) {
  if (id < c->id_base) return true;
  const uint64_t idx = id - c->id_base;
  if (idx >= c->idseq.size()) return false;
  const uint64_t v = c->idseq[idx];
  if (!v) return false;
  const uint64_t seq = v & ((1ull << 63) - 1);
  const uint32_t ring = (uint32_t)(v >> 63);
  if (seq <= completed_of(c, ring)) return true;
  // a latency-critical descriptor is seen done by its own completion word
  // before the in-order retire cursor passes it
  return ring == 1 && c->hdone_lc && load_acq(&c->hdone_lc[(seq - 1) & (c->cap - 1)]) == seq;
}

void prune_ids(gpuos_ctx* c) {
  while (!c->idseq.empty()) {
    const uint64_t v = c->idseq.front();
    if (!v) break;
    if ((v & ((1ull << 63) - 1)) > completed_of(c, (uint32_t)(v >> 63))) break;
    c->idseq.pop_front();
    ++c->id_base;
  }
}

uint32_t ring_of_id(gpuos_ctx* c, uint64_t id, bool* known) {
  *known = false;
  if (id < c->id_base) return 0;
  const uint64_t idx = id - c->id_base;
  if (idx >= c->idseq.size()) return 0;
  const uint64_t v = c->idseq[idx];
  if (v) {
    *known = true;
    return (uint32_t)(v >> 63);
  }
  for (const Staged& s : c->staged)
    if (s.id == id) {
      *known = true;
      return s.ring;
    }
  return 0;
}

// ---------------------------------------------------------------------------
// descriptor encoding

uint32_t ceil_div(uint64_t a, uint64_t b) { return (uint32_t)((a + b - 1) / b); }

// Elementwise tile: cfg.tile_elems, or be_tile_elems for ops of 2^24
// elements or more.  Large ops are cut into whole rounds over the worker
// waves (every wave gets the same number of tiles).  An op below 2^24
// elements that is big enough to give every wave 1024 elements is spread over
// all of them.  An op of 2^24 or more with fewer be_tile_elems tiles than
// waves keeps its larger tiles in the resident kernel (several such ops then
// run side by side on different waves, each tile streaming longer between
// its completion counts), with the tile count cut to a whole fraction of a
// round: k = ceil(workers / tiles) such ops fill one round, so consecutive
// ops leave no wave a tile more than the others (tiles are dealt
// round-robin); with `spread` (one launch per op, where the op is the only
// kernel running) it is spread like the others.  Tiles stay a multiple of 64
// elements so every tile starts 16-byte aligned.
uint32_t ew_tile_elems(const gpuos_config& cfg, uint32_t workers, uint64_t n, bool spread = false) {
  const bool big = n >= (1ull << 24);
  uint64_t tile = big ? cfg.be_tile_elems : cfg.tile_elems;
  uint64_t nt = (n + tile - 1) / tile;
  if (workers) {
    if (nt < workers) {
      if ((!big || spread) && n >= (uint64_t)workers * 1024) nt = workers;
      else if (big) nt = workers / ((workers + nt - 1) / nt);
    } else {
      nt = (nt + workers - 1) / workers * workers;
    }
    uint64_t t2 = (n + nt - 1) / nt;
    t2 = (t2 + 63) / 64 * 64;
    if (t2 >= 64) tile = t2;
  }
  return (uint32_t)tile;
}

void set_tiling(const gpuos_config& cfg, uint32_t workers, DevDesc& d, bool spread = false) {
  switch (d.opcode) {
    case GPUOS_OP_NOP: case GPUOS_OP_SPIN: case GPUOS_OP_ROPE:
      d.tile = 1;
      d.ntiles = 1;
      break;
    case GPUOS_OP_ROW_SUM: case GPUOS_OP_ROW_SOFTMAX: case GPUOS_OP_RMSNORM: {
      uint32_t rpt = std::max<uint32_t>(1, 4096 / d.row_len);
      const uint32_t by_waves = ceil_div(d.rows, std::max<uint32_t>(1, workers));
      rpt = std::min(rpt, std::max<uint32_t>(1, by_waves));
      d.tile = rpt;
      d.ntiles = ceil_div(d.rows, rpt);
      break;
    }
    case OP_NORM_GEMV: {
      const uint32_t units = d.ng.act ? d.ng.F : d.ng.q ? d.ng.M / 2 : d.ng.M;
      uint32_t r = ceil_div(units, std::max<uint32_t>(1, workers));
      r = std::min<uint32_t>(std::max<uint32_t>(r, 1), 16);
      d.tile = r;
      d.ntiles = ceil_div(units, r);
      break;
    }
    case GPUOS_OP_GEMV:
    case OP_GEMV_ADD: {
      // at least 2 rows per tile: a short GEMV (batch-1 projections) then
      // spends half as many waves, completion counts and dependency polls
      // on the same work, which measured faster
      const uint32_t M = (uint32_t)d.p.aux[0];
      uint32_t r = ceil_div(M, std::max<uint32_t>(1, workers));
      r = std::min<uint32_t>(std::max<uint32_t>(r, 2), 16);
      d.tile = r;
      d.ntiles = ceil_div(M, r);
      break;
    }
    case GPUOS_OP_ATTN_SCORE: {
      const uint32_t S = (uint32_t)d.p.aux[2];
      uint32_t r = ceil_div(S, std::max<uint32_t>(1, workers));
      r = std::max<uint32_t>(r, 1);
      d.tile = r;
      d.ntiles = ceil_div(S, r);
      break;
    }
    case OP_SOFTMAX_AV:  // one 8-column chunk per tile
      d.tile = 1;
      d.ntiles = (uint32_t)d.p.aux[0] * (uint32_t)d.p.aux[1] / 8;
      break;
    case GPUOS_OP_ATTN_AV: {
      const uint32_t H = (uint32_t)d.p.aux[0], D = (uint32_t)d.p.aux[1];
      if (D % 8 == 0) {
        d.tile = 1;
        d.ntiles = H * D / 8;
      } else {
        d.tile = 8;
        d.ntiles = ceil_div((uint64_t)H * D, 8);
      }
      break;
    }
    default: {  // elementwise and fused
      d.tile = ew_tile_elems(cfg, workers, d.n, spread);
      d.ntiles = ceil_div(d.n, d.tile);
      break;
    }
  }
}

void encode_plain(const gpuos_op& o, const gpuos_config& cfg, uint32_t workers, DevDesc& d,
                  bool spread = false) {
  memset(&d, 0, sizeof d);
  d.opcode = (uint8_t)o.opcode;
  d.dtype = o.dtype;
  d.flags = o.flags;
  d.n = o.n;
  d.rows = o.rows;
  d.row_len = o.row_len;
  if (o.opcode == GPUOS_OP_GATHER || o.opcode == GPUOS_OP_NOP || o.opcode == GPUOS_OP_SPIN) {
    // nothing to normalise
  }
  d.p.ptr[0] = (uint64_t)o.out;
  d.p.ptr[1] = (uint64_t)o.in[0];
  d.p.ptr[2] = (uint64_t)o.in[1];
  d.p.ptr[3] = (uint64_t)o.in[2];
  for (int i = 0; i < 2; ++i) {
    uint64_t sl = o.src_len[i];
    if (o.opcode != GPUOS_OP_GATHER && sl >= o.n) sl = 0;  // a longer source is read as a prefix
    d.p.src_len[i] = (uint32_t)sl;
  }
  d.p.alpha = o.alpha;
  d.p.eps = o.eps;
  for (int i = 0; i < 4; ++i) d.p.aux[i] = o.aux[i];
  if (o.opcode == GPUOS_OP_ROPE) {
    d.rows = o.rows;
    d.row_len = o.row_len;
  }
  d.user_ops = 1;
  set_tiling(cfg, workers, d, spread);
}

// ---------------------------------------------------------------------------
// fusion pass: merges maximal runs of adjacent elementwise ops in which each
// op consumes its predecessor's output element for element into one
// FUSED_EW descriptor ("Launch Overhead and Fusion", section "Fusion": one
// pass, intermediates kept in registers).  Results stay bit-identical: every
// step is the same single IEEE operation, rounded to the storage type after
// each step, and stores of intermediates are kept unless the op is marked
// transient and no later queued op reads it.

uint8_t fuse_code(uint32_t op) {
  switch (op) {
    case GPUOS_OP_ADD: return FS_ADD;
    case GPUOS_OP_MUL: return FS_MUL;
    case GPUOS_OP_SCALE: return FS_SCALE;
    case GPUOS_OP_RELU: return FS_RELU;
    case GPUOS_OP_EXP: return FS_EXP;
    case GPUOS_OP_COPY: return FS_COPY;
    default: return 0;
  }
}

bool fusable(const gpuos_op& o) {
  if (!fuse_code(o.opcode)) return false;
  // fp32 chains only: a bf16 chain would re-round after every step in
  // registers, and its register footprint would cap the resident kernel's
  // occupancy for every other op
  if (o.dtype != GPUOS_F32) return false;
  if (o.src_len[0] && o.src_len[0] < o.n) return false;
  if (is_binary(o.opcode) && o.src_len[1] && o.src_len[1] < o.n) return false;
  return true;
}

struct ChainState {
  uint64_t chain_in = 0;           // pointer loaded into the accumulator
  uint64_t operands[3] = {0, 0, 0};
  int nops = 0;
  SmallVec<Range, kMaxSteps> outs;   // output ranges written so far (in order)
  SmallVec<Range, 4> reads;          // every range read by the chain
  uint64_t last_out = 0;
};

// Can op `o` extend the chain whose previous op wrote `st.last_out`?
// On success fills the step encoding.
bool try_extend(const gpuos_op& o, ChainState& st, uint8_t& code, uint8_t& fl) {
  const uint64_t es = elem_size(o.dtype);
  const uint64_t bytes = (uint64_t)o.n * es;
  const uint64_t P = st.last_out;
  const uint64_t i0 = (uint64_t)o.in[0], i1 = (uint64_t)o.in[1];
  code = fuse_code(o.opcode);
  fl = 0;
  uint64_t operand = 0;
  if (is_binary(o.opcode)) {
    if (i0 == P && i1 == P)
      fl = FSF_SELF;
    else if (i0 == P)
      operand = i1;
    else if (i1 == P)
      operand = i0;
    else
      return false;
  } else {
    if (i0 != P) return false;
  }
  const Range out{(uint64_t)o.out, (uint64_t)o.out + bytes};
  if (operand) {
    const Range orng{operand, operand + bytes};
    // the operand is loaded before any step runs: it must not depend on a
    // value written earlier in the chain
    for (const Range& w : st.outs)
      if (overlaps(w, orng)) return false;
  }
  // the new output must not clobber, at another element, anything the chain
  // reads; in place (same base) is fine because loads precede stores
  auto ok_against = [&](const Range& r) {
    return !overlaps(r, out) || r.lo == out.lo;
  };
  for (const Range& r : st.reads)
    if (!ok_against(r)) return false;
  for (const Range& w : st.outs)
    if (overlaps(w, out) && w.lo != out.lo) return false;
  if (operand) {
    const Range orng{operand, operand + bytes};
    if (!ok_against(orng)) return false;
    int idx = -1;
    for (int k = 0; k < st.nops; ++k)
      if (st.operands[k] == operand) idx = k;
    if (idx < 0) {
      if (st.nops == 3) return false;
      idx = st.nops;
      st.operands[st.nops++] = operand;
    }
    fl |= (uint8_t)(FSF_OPERAND | ((idx + 1) << 4));
    st.reads.push_back(orng);
  }
  st.outs.push_back(out);
  st.last_out = (uint64_t)o.out;
  return true;
}

// Puts a PROGRAM op's body into its descriptor (over the plain op's
// src_len, scalar and aux fields, which such an op does not use).
void encode_program(const ProgCode& pc, DevDesc& d) {
  d.pg.meta = pc.meta;
  for (int s = 0; s < GPUOS_PROG_MAX_INSNS; ++s) d.pg.ins[s] = pc.ins[s];
  for (int j = 0; j < 8; ++j) d.pg.k[j] = pc.k[j];
}

// A latency-critical op is run by the one reserved wave that claims its
// descriptor, tile after tile; a small elementwise, COPY, fused or PROGRAM
// op (plain layout, up to 2^16 elements) becomes a single tile, which that
// wave streams with its loads pipelined and completes without a counter.
constexpr uint32_t kLcOneTileElems = 1u << 16;

void one_tile_if_small(DevDesc& d) {
  if (d.flags & DF_VIEW) return;
  const bool stream = d.opcode == OP_FUSED_EW || d.opcode == GPUOS_OP_PROGRAM ||
                      (is_elementwise(d.opcode) && d.opcode != GPUOS_OP_GATHER);
  if (stream && d.n <= kLcOneTileElems) {
    d.tile = d.n;
    d.ntiles = 1;
  }
}

// Streams (non-temporal) elementwise, COPY, fused and PROGRAM descriptors
// whose operands total at least stream_min_kib.
void mark_streaming(const gpuos_config& cfg, DevDesc& d) {
  if (cfg.stream_min_kib == 0xFFFFFFFFu || (d.flags & DF_VIEW)) return;
  const uint64_t es = elem_size(d.dtype);
  uint64_t bytes = 0;
  if (d.opcode == OP_FUSED_EW) {
    uint32_t k = 0;
    for (int i = 0; i < 4; ++i) k += d.f.in[i] != 0;
    for (int i = 0; i < kMaxSteps; ++i) k += d.f.out[i] != 0;
    bytes = (uint64_t)k * d.n * es;
  } else if (d.opcode == GPUOS_OP_PROGRAM) {
    bytes = (uint64_t)(1 + ((d.pg.meta >> 16) & 3u)) * d.n * es;
  } else if (is_elementwise(d.opcode) && d.opcode != GPUOS_OP_GATHER) {
    const uint64_t ext = (uint64_t)d.n * es;
    const uint64_t l0 = d.p.src_len[0] ? std::min<uint64_t>(d.p.src_len[0], d.n) * es : ext;
    const uint64_t l1 = d.p.src_len[1] ? std::min<uint64_t>(d.p.src_len[1], d.n) * es : ext;
    bytes = ext + (d.p.ptr[1] ? l0 : 0) + (d.p.ptr[2] && is_binary(d.opcode) ? l1 : 0);
  } else {
    return;
  }
  if (bytes >= (uint64_t)cfg.stream_min_kib * 1024) d.flags |= GPUOS_FLAG_NONTEMPORAL;
}

// Adds an elementwise op's view to its descriptor: rows of shape[3]
// elements, about 1,024 elements per tile, spread over the workers.
void encode_view(const ViewDesc& v, uint32_t workers, DevDesc& d) {
  d.flags = (uint8_t)((d.flags | DF_VIEW) & ~GPUOS_FLAG_NONTEMPORAL);
  for (int j = 0; j < 4; ++j) {
    d.p.vshape[j] = v.shape[j];
    for (int k = 0; k < 3; ++k) d.p.vstride[k][j] = (int32_t)v.stride[k][j];
  }
  const uint64_t rows = (uint64_t)v.shape[0] * v.shape[1] * v.shape[2], L = v.shape[3];
  // a (batched) 2-D transposing COPY: per batch, blocks of 128 / element
  // size rows by kTCols columns
  if (d.opcode == GPUOS_OP_COPY && v.shape[0] == 1 && v.stride[0][3] == 1 && v.stride[1][2] == 1 &&
      v.stride[1][3] > 1) {
    const uint64_t K = kTBlockBytes / elem_size(d.dtype), R = v.shape[2];
    d.flags |= DF_VIEW_T;
    d.tile = (uint32_t)K;
    d.ntiles = (uint32_t)(v.shape[1] * ((R + K - 1) / K) * ((L + kTCols - 1) / kTCols));
    return;
  }
  uint64_t nt = std::max<uint64_t>(1, (rows * L + 1023) / 1024);
  nt = std::min<uint64_t>(nt, std::max<uint32_t>(1, workers));
  nt = std::min<uint64_t>(nt, rows);
  d.tile = (uint32_t)((rows + nt - 1) / nt);
  d.ntiles = (uint32_t)((rows + d.tile - 1) / d.tile);
}

// Is output range `w` of staged op `from` - 1 read by any op staged after it?
bool read_later(gpuos_ctx* c, size_t from, const Range& w) {
  for (size_t k = from; k < c->staged.size(); ++k) {
    const OpRanges R = op_ranges(c->staged[k].op, &c->staged[k].view);
    for (int q = 0; q < R.nr; ++q)
      if (overlaps(R.r[q], w)) return true;
  }
  return false;
}

// RMSNORM (one bf16 row of K) -> GEMV on that row (K <= 1,024) -> optionally
// SILU_MUL on the two halves of the GEMV output: fused into one descriptor
// when the ops are adjacent, in one ring, 16-byte aligned, and no output
// overlaps an input of the group (tiles run concurrently).  Returns the
// number of user ops fused (0 = none).
uint32_t try_norm_gemv(gpuos_ctx* c, size_t i, size_t end, DevDesc& d) {
  if (i + 1 >= end) return 0;
  const Staged& sa = c->staged[i];
  const Staged& sb = c->staged[i + 1];
  const gpuos_op& A = sa.op;
  const gpuos_op& B = sb.op;
  if (A.opcode != GPUOS_OP_RMSNORM || B.opcode != GPUOS_OP_GEMV) return 0;
  if (A.dtype != GPUOS_BF16 || B.dtype != GPUOS_BF16 || sa.ring != sb.ring) return 0;
  const uint32_t K = A.row_len, M = (uint32_t)B.aux[0];
  if (A.rows != 1 || (uint32_t)B.aux[1] != K || K % 8 || K > 1024 || B.in[0] != A.out) return 0;
  if (A.src_len[0] && A.src_len[0] < K) return 0;
  const uint64_t x = (uint64_t)A.in[0], g = (uint64_t)A.in[2], h = (uint64_t)A.out;
  const uint64_t W = (uint64_t)B.in[2], y = (uint64_t)B.out;
  for (uint64_t p : {x, g, h, W, y})
    if (p % 16) return 0;
  const Range rx{x, x + 2ull * K}, rg{g, g + 2ull * K}, rh{h, h + 2ull * K};
  const Range rW{W, W + 2ull * M * K}, ry{y, y + 2ull * M};
  for (const Range& o : {rh, ry})
    for (const Range& in : {rx, rg, rW})
      if (overlaps(o, in)) return 0;
  if (overlaps(rh, ry)) return 0;
  uint32_t count = 2;
  uint64_t act = 0;
  uint32_t F = 0;
  if (i + 2 < end) {
    const Staged& sc = c->staged[i + 2];
    const gpuos_op& C = sc.op;
    const uint32_t f = M / 2;
    if (C.opcode == GPUOS_OP_SILU_MUL && C.dtype == GPUOS_BF16 && sc.ring == sa.ring && !sc.view.on &&
        M % 2 == 0 && C.n == f && (uint64_t)C.in[0] == y && (uint64_t)C.in[1] == y + 2ull * f &&
        (!C.src_len[0] || C.src_len[0] >= f) && (!C.src_len[1] || C.src_len[1] >= f)) {
      const Range ra{(uint64_t)C.out, (uint64_t)C.out + 2ull * f};
      bool clear = !overlaps(ra, ry);
      for (const Range& in : {rx, rg, rW, rh})
        if (overlaps(ra, in)) clear = false;
      if (clear) {
        act = (uint64_t)C.out;
        F = f;
        count = 3;
      }
    }
  }
  // rotary mode: ROPE of the q third, ROPE of the k third, COPY of the v third
  uint64_t rq = 0, rk = 0, rv = 0, tq = 0, tk = 0;
  uint32_t hd = 0;
  if (!F && i + 4 < end) {
    const gpuos_op& Q = c->staged[i + 2].op;
    const gpuos_op& Kr = c->staged[i + 3].op;
    const gpuos_op& Cv = c->staged[i + 4].op;
    bool ok = c->staged[i + 2].ring == sa.ring && c->staged[i + 3].ring == sa.ring &&
              c->staged[i + 4].ring == sa.ring && !c->staged[i + 4].view.on && Q.opcode == GPUOS_OP_ROPE &&
              Kr.opcode == GPUOS_OP_ROPE && Cv.opcode == GPUOS_OP_COPY && Q.dtype == GPUOS_BF16 &&
              Kr.dtype == GPUOS_BF16 && Cv.dtype == GPUOS_BF16;
    const uint32_t H = Q.rows, h = Q.row_len, Dq = H * h;
    ok = ok && h >= 2 && h % 2 == 0 && Kr.rows == H && Kr.row_len == h && Cv.n == Dq &&
         M == 3 * Dq && (uint64_t)Q.in[0] == y && (uint64_t)Kr.in[0] == y + 2ull * Dq &&
         (uint64_t)Cv.in[0] == y + 4ull * Dq;
    for (const gpuos_op* o : {&Q, &Kr, &Cv})
      ok = ok && (!o->src_len[0] || o->src_len[0] >= o->n);
    if (ok) {
      const Range oq{(uint64_t)Q.out, (uint64_t)Q.out + 2ull * Dq};
      const Range ok_{(uint64_t)Kr.out, (uint64_t)Kr.out + 2ull * Dq};
      const Range ov{(uint64_t)Cv.out, (uint64_t)Cv.out + 2ull * Dq};
      const Range rtq{(uint64_t)Q.in[2], (uint64_t)Q.in[2] + 4ull * h};
      const Range rtk{(uint64_t)Kr.in[2], (uint64_t)Kr.in[2] + 4ull * h};
      for (const Range& o : {oq, ok_, ov}) {
        for (const Range& in : {rx, rg, rW, rh, ry, rtq, rtk})
          if (overlaps(o, in)) ok = false;
      }
      if (overlaps(oq, ok_) || overlaps(oq, ov) || overlaps(ok_, ov)) ok = false;
      if (ok) {
        rq = (uint64_t)Q.out;
        rk = (uint64_t)Kr.out;
        rv = (uint64_t)Cv.out;
        tq = (uint64_t)Q.in[2];
        tk = (uint64_t)Kr.in[2];
        hd = h;
        count = 5;
      }
    }
  }
  memset(&d, 0, sizeof d);
  d.opcode = OP_NORM_GEMV;
  d.dtype = GPUOS_BF16;
  d.flags = (uint8_t)((B.flags & DF_AUX_READY) | ((A.flags | B.flags) & GPUOS_FLAG_NONTEMPORAL));
  d.n = F ? F : M;
  d.ng.W = W;
  d.ng.x = x;
  d.ng.g = g;
  // intermediates are stored unless transient and unread by later ops
  const bool keep_h = !(A.flags & GPUOS_FLAG_TRANSIENT) || read_later(c, i + count, rh);
  const bool keep_y = (!F && !rq) || !(B.flags & GPUOS_FLAG_TRANSIENT) || read_later(c, i + count, ry);
  d.ng.h = keep_h ? h : 0;
  d.ng.out = keep_y ? y : 0;
  d.ng.act = act;
  d.ng.M = M;
  d.ng.K = K;
  d.ng.eps = A.eps;
  d.ng.F = F;
  d.ng.q = rq;
  d.ng.k = rk;
  d.ng.v = rv;
  d.ng.tabq = tq;
  d.ng.tabk = tk;
  d.ng.hd = hd;
  d.user_ops = count;
  set_tiling(c->cfg, c->workers, d);
  return count;
}

// GEMV -> ADD of that GEMV's output (read at the same index) and a residual,
// same dtype, n == M: one descriptor whose tiles finish each output row with
// the add.  The ADD may write the residual in place (each element is read
// and written by the wave that owns its row) but its output may not overlap
// any other operand, and the GEMV output may not overlap x, W or the
// residual.  Returns the number of user ops fused (0 = none).
uint32_t try_gemv_add(gpuos_ctx* c, size_t i, size_t end, DevDesc& d) {
  if (i + 1 >= end) return 0;
  const Staged& sa = c->staged[i];
  const Staged& sb = c->staged[i + 1];
  const gpuos_op& A = sa.op;
  const gpuos_op& B = sb.op;
  if (A.opcode != GPUOS_OP_GEMV || B.opcode != GPUOS_OP_ADD || sa.ring != sb.ring || sb.view.on) return 0;
  if (A.dtype != B.dtype || (A.dtype != GPUOS_F32 && A.dtype != GPUOS_BF16)) return 0;
  const uint32_t M = (uint32_t)A.aux[0], K = (uint32_t)A.aux[1];
  if (B.n != M) return 0;
  const uint64_t y = (uint64_t)A.out;
  bool res_first;
  if ((uint64_t)B.in[1] == y && (uint64_t)B.in[0] != y)
    res_first = true;
  else if ((uint64_t)B.in[0] == y && (uint64_t)B.in[1] != y)
    res_first = false;
  else
    return 0;
  for (int q = 0; q < 2; ++q)
    if (B.src_len[q] && B.src_len[q] < M) return 0;  // cyclic reads stay unfused
  const uint64_t es = elem_size(A.dtype);
  const uint64_t x = (uint64_t)A.in[0], W = (uint64_t)A.in[2];
  const uint64_t r = (uint64_t)(res_first ? B.in[0] : B.in[1]), z = (uint64_t)B.out;
  const Range rx{x, x + es * K}, rW{W, W + 2ull * M * K}, ry{y, y + es * M};
  const Range rr{r, r + es * M}, rz{z, z + es * M};
  for (const Range& in : {rx, rW, rr})
    if (overlaps(ry, in)) return 0;
  for (const Range& in : {rx, rW, ry})
    if (overlaps(rz, in)) return 0;
  if (overlaps(rz, rr) && z != r) return 0;
  memset(&d, 0, sizeof d);
  d.opcode = OP_GEMV_ADD;
  d.dtype = A.dtype;
  d.flags = (uint8_t)((A.flags & DF_AUX_READY) | ((A.flags | B.flags) & GPUOS_FLAG_NONTEMPORAL));
  d.n = M;
  // the GEMV output is stored unless transient and unread by later ops
  const bool keep_y = !(A.flags & GPUOS_FLAG_TRANSIENT) || read_later(c, i + 2, ry);
  d.ga.out = keep_y ? y : 0;
  d.ga.x = x;
  d.ga.res = r;
  d.ga.W = W;
  d.ga.res_first = res_first ? 1u : 0u;
  d.ga.M = M;
  d.ga.K = K;
  d.ga.sum = z;
  d.user_ops = 2;
  set_tiling(c->cfg, c->workers, d);
  return 2;
}

// ROW_SOFTMAX over fp32 score rows -> ATTN_AV reading those probabilities:
// one descriptor whose AV tiles each compute their head's softmax row (rows
// of at most 512 elements, a multiple of 4; head size a multiple of 8;
// scores, probabilities and V 16-byte aligned; no output overlapping an
// input).  The probabilities are stored unless transient and unread later.
uint32_t try_softmax_av(gpuos_ctx* c, size_t i, size_t end, DevDesc& d) {
  if (i + 1 >= end) return 0;
  const Staged& sa = c->staged[i];
  const Staged& sb = c->staged[i + 1];
  const gpuos_op& A = sa.op;
  const gpuos_op& B = sb.op;
  if (A.opcode != GPUOS_OP_ROW_SOFTMAX || B.opcode != GPUOS_OP_ATTN_AV || sa.ring != sb.ring) return 0;
  if (A.dtype != GPUOS_F32 || (B.dtype != GPUOS_F32 && B.dtype != GPUOS_BF16)) return 0;
  const uint32_t H = (uint32_t)B.aux[0], Dh = (uint32_t)B.aux[1], S = (uint32_t)B.aux[2];
  if (A.rows != H || A.row_len != S || S % 4 || S > 4 * 128 || Dh % 8) return 0;
  if (A.src_len[0] && A.src_len[0] < A.n) return 0;
  const uint64_t x = (uint64_t)A.in[0], p = (uint64_t)A.out, V = (uint64_t)B.in[2];
  const uint64_t o = (uint64_t)B.out;
  if ((uint64_t)B.in[0] != p || x % 16 || p % 16 || V % 16) return 0;
  const uint64_t rowsb = 4ull * H * S;
  const Range rx{x, x + rowsb}, rp{p, p + rowsb}, rV{V, V + 2ull * S * H * Dh};
  const Range ro{o, o + elem_size(B.dtype) * H * Dh};
  for (const Range& in : {rx, rV})
    if (overlaps(rp, in) || overlaps(ro, in)) return 0;
  if (overlaps(rp, ro)) return 0;
  memset(&d, 0, sizeof d);
  d.opcode = OP_SOFTMAX_AV;
  d.dtype = B.dtype;
  d.flags = (uint8_t)((A.flags | B.flags) & GPUOS_FLAG_NONTEMPORAL);
  d.n = H * Dh;
  const bool keep_p = !(A.flags & GPUOS_FLAG_TRANSIENT) || read_later(c, i + 2, rp);
  d.p.ptr[0] = o;
  d.p.ptr[1] = keep_p ? p : 0;
  d.p.ptr[2] = x;
  d.p.ptr[3] = V;
  d.p.aux[0] = (int32_t)H;
  d.p.aux[1] = (int32_t)Dh;
  d.p.aux[2] = (int32_t)S;
  d.user_ops = 2;
  set_tiling(c->cfg, c->workers, d);
  return 2;
}

// A PROGRAM op whose body is a chain over one accumulator, in fp32, can run as
// the built-in op or fused micro-program that performs the same fp32
// operations in the same order: each instruction reads the accumulator (the
// previous instruction's result, first an input register) and at most an
// unwritten input register, the accumulator again, or, for MUL, a constant
// (then a SCALE step), and the result is the last accumulator.  ADD and MUL
// are commutative in IEEE arithmetic, so acc + x and x + acc are the same
// result.  This is the operators compiled at run time of the pages, for the
// programs the fused tile can express; any other program is interpreted.
bool program_as_builtin(const Staged& st, const gpuos_config& cfg, uint32_t workers, DevDesc& d,
                        bool spread = false) {
  const gpuos_op& o = st.op;
  if (o.dtype != GPUOS_F32) return false;
  const ProgCode& pc = st.prog;
  const uint32_t ni = pc.meta & 31u, res = (pc.meta >> 8) & 15u, nin = pc.n_inputs();
  if (ni > (uint32_t)kMaxSteps) return false;
  const uint64_t inp[3] = {(uint64_t)o.in[0], (uint64_t)o.in[1], (uint64_t)o.in[2]};
  uint32_t written = 0;
  int acc = -1;
  uint64_t chain_in = 0, operands[3] = {0, 0, 0};
  int nops = 0;
  uint8_t codes[kMaxSteps], fls[kMaxSteps];
  float scal[kMaxSteps];
  uint32_t opnd_reg[kMaxSteps];
  auto is_input = [&](uint32_t r) { return r < nin && !(written & (1u << r)); };
  for (uint32_t s = 0; s < ni; ++s) {
    const uint32_t w = pc.ins[s], op = w & 31u, dst = (w >> 5) & 7u;
    uint32_t a = (w >> 8) & 15u, b = (w >> 12) & 15u;
    const bool binary = op == GPUOS_P_ADD || op == GPUOS_P_MUL;
    if (acc < 0) {  // the chain starts from an input register
      if (!is_input(a)) {
        if (!binary || !is_input(b)) return false;
        std::swap(a, b);
      }
      chain_in = inp[a];
      acc = (int)a;
    }
    uint8_t code = 0, fl = 0;
    float k = 0.0f;
    opnd_reg[s] = 0;
    switch (op) {
      case GPUOS_P_MOV: case GPUOS_P_RELU: case GPUOS_P_EXP:
        if ((int)a != acc) return false;
        code = op == GPUOS_P_MOV ? FS_COPY : op == GPUOS_P_RELU ? FS_RELU : FS_EXP;
        break;
      case GPUOS_P_ADD: case GPUOS_P_MUL: {
        uint32_t other;
        if ((int)a == acc) other = b;
        else if ((int)b == acc) other = a;
        else return false;
        code = op == GPUOS_P_ADD ? FS_ADD : FS_MUL;
        if ((int)other == acc) {
          fl = FSF_SELF;
        } else if (is_input(other)) {
          int slot = 0;
          for (int q = 0; q < nops; ++q)
            if (operands[q] == inp[other]) slot = q + 1;
          if (!slot) {
            if (nops == 3) return false;
            operands[nops++] = inp[other];
            slot = nops;
          }
          fl = (uint8_t)(FSF_OPERAND | (slot << 4));
          opnd_reg[s] = other;
        } else if (other >= 8 && op == GPUOS_P_MUL) {
          code = FS_SCALE;
          k = pc.k[other - 8];
        } else {
          return false;
        }
        break;
      }
      default:
        return false;
    }
    codes[s] = code;
    fls[s] = fl;
    scal[s] = k;
    written |= 1u << dst;
    acc = (int)dst;
  }
  if ((int)res != acc) return false;
  if (ni == 1) {  // one step: the plain built-in op
    gpuos_op po;
    memset(&po, 0, sizeof po);
    po.dtype = GPUOS_F32;
    po.flags = o.flags;
    po.n = o.n;
    po.out = o.out;
    po.in[0] = (const void*)chain_in;
    switch (codes[0]) {
      case FS_ADD: case FS_MUL:
        po.opcode = codes[0] == FS_ADD ? GPUOS_OP_ADD : GPUOS_OP_MUL;
        po.in[1] = (fls[0] & FSF_SELF) ? (const void*)chain_in : (const void*)inp[opnd_reg[0]];
        break;
      case FS_SCALE: po.opcode = GPUOS_OP_SCALE; po.alpha = scal[0]; break;
      case FS_RELU: po.opcode = GPUOS_OP_RELU; break;
      case FS_EXP: po.opcode = GPUOS_OP_EXP; break;
      default: po.opcode = GPUOS_OP_COPY; break;
    }
    encode_plain(po, cfg, workers, d, spread);
    return true;
  }
  memset(&d, 0, sizeof d);
  d.opcode = OP_FUSED_EW;
  d.dtype = GPUOS_F32;
  d.flags = (uint8_t)(o.flags & GPUOS_FLAG_NONTEMPORAL);
  d.n = o.n;
  d.nsteps = (uint8_t)ni;
  d.f.in[0] = chain_in;
  for (int q = 0; q < 3; ++q) d.f.in[q + 1] = operands[q];
  for (uint32_t s = 0; s < ni; ++s) {
    d.f.step_op[s] = codes[s];
    d.f.fscal[s] = scal[s];
    d.f.step_fl[s] = fls[s];
  }
  d.f.out[ni - 1] = (uint64_t)o.out;
  d.f.step_fl[ni - 1] = (uint8_t)(fls[ni - 1] | FSF_STORE);
  d.user_ops = 1;
  set_tiling(cfg, workers, d, spread);
  return true;
}

void plan_ops(gpuos_ctx* c, size_t begin, size_t end, std::vector<Planned>& plan) {
  const gpuos_config& cfg = c->cfg;
  const bool fuse = cfg.fusion == 1;
  size_t i = begin;
  while (i < end) {
    const Staged& s0 = c->staged[i];
    Planned& pl = plan.emplace_back();
    pl.first = i;
    pl.count = 1;
    pl.ring = s0.ring;
    pl.deps.clear();
    size_t j = i + 1;
    if (fuse) {
      uint32_t k = try_norm_gemv(c, i, end, pl.desc);
      if (!k) k = try_gemv_add(c, i, end, pl.desc);
      if (!k) k = try_softmax_av(c, i, end, pl.desc);
      if (k) {
        pl.count = k;
        c->st.ops_fused += k - 1;
      }
    }
    // a chain needs a next op of the same ring, dtype and size that reads
    // this op's output
    bool chain_possible = false;
    if (pl.count == 1 && fuse && j < end && fusable(s0.op) && !s0.view.on) {
      const gpuos_op& nx = c->staged[j].op;
      chain_possible = c->staged[j].ring == s0.ring && fusable(nx) && !c->staged[j].view.on &&
                       nx.dtype == s0.op.dtype &&
                       nx.n == s0.op.n && (nx.in[0] == s0.op.out || nx.in[1] == s0.op.out);
    }
    if (chain_possible) {
      ChainState st;
      const gpuos_op& o0 = s0.op;
      const uint64_t es = elem_size(o0.dtype);
      const uint64_t bytes = (uint64_t)o0.n * es;
      st.chain_in = (uint64_t)o0.in[0];
      st.reads.push_back(Range{st.chain_in, st.chain_in + bytes});
      uint8_t fl0 = 0;
      if (is_binary(o0.opcode)) {
        if (o0.in[1] == o0.in[0]) {
          fl0 = FSF_SELF;
        } else {
          st.operands[0] = (uint64_t)o0.in[1];
          st.nops = 1;
          fl0 = (uint8_t)(FSF_OPERAND | (1 << 4));
          st.reads.push_back(Range{st.operands[0], st.operands[0] + bytes});
        }
      }
      const Range out0{(uint64_t)o0.out, (uint64_t)o0.out + bytes};
      bool first_ok = true;
      for (const Range& r : st.reads)
        if (overlaps(r, out0) && r.lo != out0.lo) first_ok = false;
      if (first_ok) {
        st.outs.push_back(out0);
        st.last_out = (uint64_t)o0.out;
        uint8_t codes[kMaxSteps], fls[kMaxSteps];
        codes[0] = fuse_code(o0.opcode);
        fls[0] = fl0;
        uint32_t n_steps = 1;
        const uint32_t max_steps = std::min<uint32_t>(cfg.max_fuse, kMaxSteps);
        while (j < end && n_steps < max_steps) {
          const Staged& sj = c->staged[j];
          if (sj.ring != s0.ring || !fusable(sj.op) || sj.view.on || sj.op.dtype != o0.dtype ||
              sj.op.n != o0.n)
            break;
          ChainState trial = st;
          uint8_t code, fl;
          if (!try_extend(sj.op, trial, code, fl)) break;
          st = trial;
          codes[n_steps] = code;
          fls[n_steps] = fl;
          ++n_steps;
          ++j;
        }
        if (n_steps > 1) {
          DevDesc& d = pl.desc;
          memset(&d, 0, sizeof d);
          d.opcode = OP_FUSED_EW;
          d.dtype = o0.dtype;
          d.n = o0.n;
          d.nsteps = (uint8_t)n_steps;
          d.f.in[0] = st.chain_in;
          for (int k = 0; k < 3; ++k) d.f.in[k + 1] = st.operands[k];
          for (uint32_t s = 0; s < n_steps; ++s) {
            const gpuos_op& os = c->staged[i + s].op;
            d.f.step_op[s] = codes[s];
            d.f.fscal[s] = os.alpha;
            d.flags |= (uint8_t)(os.flags & GPUOS_FLAG_NONTEMPORAL);
            // keep the store unless the op is transient and nothing queued
            // after the chain reads its output
            bool keep = !(os.flags & GPUOS_FLAG_TRANSIENT);
            if (!keep) {
              const Range w{(uint64_t)os.out, (uint64_t)os.out + bytes};
              for (size_t k = j; k < c->staged.size() && !keep; ++k) {
                const OpRanges R = op_ranges(c->staged[k].op, &c->staged[k].view);
                for (int q = 0; q < R.nr; ++q)
                  if (overlaps(R.r[q], w)) keep = true;
              }
            }
            d.f.out[s] = keep ? (uint64_t)os.out : 0;
            d.f.step_fl[s] = (uint8_t)(fls[s] | (keep ? FSF_STORE : 0));
          }
          d.user_ops = n_steps;
          set_tiling(cfg, c->workers, d, c->spread_big);
          pl.count = n_steps;
          c->st.ops_fused += n_steps - 1;
        }
      }
    }
    if (pl.count == 1) {
      if (s0.op.opcode == GPUOS_OP_PROGRAM && fuse && program_as_builtin(s0, cfg, c->workers, pl.desc, c->spread_big)) {
        ++c->st.programs_lowered;
      } else {
        encode_plain(s0.op, cfg, c->workers, pl.desc, c->spread_big);
        if (s0.view.on) encode_view(s0.view, c->workers, pl.desc);
        if (s0.op.opcode == GPUOS_OP_PROGRAM) {
          encode_program(s0.prog, pl.desc);
          // the latest compiled variant's body for it, if any
          const RtcModule* m = c->rtc_new.get();
          if (m && ((m->dtypes >> pl.desc.dtype) & 1u)) {
            const auto it = m->index.find(body_key(s0.prog));
            if (it != m->index.end()) pl.desc.pg.body = it->second + 1;
          }
        }
      }
      j = i + 1;
    }
    mark_streaming(cfg, pl.desc);
    if (pl.ring == 1) one_tile_if_small(pl.desc);
    // dependencies: union of the members' deps that point outside the group
    const uint64_t gfirst = c->staged[i].id, glast = c->staged[i + pl.count - 1].id;
    for (uint32_t k = 0; k < pl.count; ++k)
      for (uint64_t dep : c->staged[i + k].deps)
        if (dep < gfirst || dep > glast) pl.deps.push_back(dep);
    pl.deps.sort_unique();
    i = i + pl.count;
  }
}

// Launches the resident kernel (epoch + 1), its first ring-0 ticket `base`.
// HIP events recorded just before and just after the launch on its stream
// bracket exactly that launch.
int launch_kernel(gpuos_ctx* c, uint64_t base) {
  c->kargs.epoch = ++c->epoch;
  c->kargs.ticket_base = base;
  hipError_t e = hipEventRecord(c->ev_start, c->stream);
  if (e == hipSuccess) {
    if (c->on_rtc) {
      void* args[] = {&c->kargs};
      e = hipModuleLaunchKernel(c->rtc_run->fn, c->blocks, 1, 1, 256, 1, 1, 0, c->stream, args, nullptr);
    } else {
      e = launch_resident(c->kargs, c->blocks, c->stream);
    }
  }
  if (e == hipSuccess) e = hipEventRecord(c->ev_end, c->stream);
  if (e != hipSuccess) {
    c->poisoned = true;
    c->exited = true;
    return fail(GPUOS_EDEVICE, "resident launch: %s", hipGetErrorString(e));
  }
  c->timing = true;
  ++c->st.launches;
  return 0;
}

// Adds the duration of the last launch, which has ended, to kernel_ns.
void account_launch(gpuos_ctx* c) {
  if (!c->timing) return;
  c->timing = false;
  float ms = 0.0f;
  if (hipEventSynchronize(c->ev_end) == hipSuccess &&
      hipEventElapsedTime(&ms, c->ev_start, c->ev_end) == hipSuccess)
    c->st.kernel_ns += (uint64_t)((double)ms * 1e6);
}

// Waits (bounded) for the resident kernel's launch to end.
int wait_kernel_end(gpuos_ctx* c, int64_t timeout_ns) {
  const auto t0 = std::chrono::steady_clock::now();
  for (;;) {
    const hipError_t e = hipStreamQuery(c->stream);
    if (e == hipSuccess) return 0;
    if (e != hipErrorNotReady) {
      c->exited = true;
      c->poisoned = true;
      return fail(GPUOS_EDEVICE, "resident kernel failed: %s", hipGetErrorString(e));
    }
    if (timeout_ns >= 0 &&
        std::chrono::steady_clock::now() - t0 > std::chrono::nanoseconds(timeout_ns)) {
      c->leaked = true;
      return fail(GPUOS_ETIMEDOUT, "resident kernel did not exit");
    }
    std::this_thread::sleep_for(std::chrono::microseconds(20));
  }
}

// Waits until every wave of the launch just made has started (the doorbell
// wave publishes resident_epoch once the grid has checked in).  If that does
// not happen within 10 s, the kernel is told to stop (it leaves without
// taking work) and the context fails.
int wait_resident(gpuos_ctx* c) {
  const auto t0 = std::chrono::steady_clock::now();
  while (load_acq(&c->hctl->resident_epoch) != c->epoch) {
    const hipError_t e = hipStreamQuery(c->stream);
    if (e != hipErrorNotReady) {
      c->poisoned = true;
      c->exited = true;
      return fail(GPUOS_EDEVICE, "resident kernel ended before its grid was resident: %s",
                  hipGetErrorString(e));
    }
    if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(10)) {
      c->poisoned = true;
      store_rel(&c->hctl->stop_req, 1);
      if (wait_kernel_end(c, 2ll * 1000 * 1000 * 1000) == 0) c->exited = true;
      else c->leaked = true;  // still running: its memory must not be freed
      return fail(GPUOS_EDEVICE, "the resident grid of %u waves did not become resident within 10 s "
                  "(another kernel may hold compute units)", c->blocks * 4);
    }
    std::this_thread::sleep_for(std::chrono::microseconds(20));
  }
  return 0;
}

// Called from every host wait and after every flush: if the kernel has left
// after an idle period, waits for its launch to end and launches it again.
// A kernel that ended without announcing an exit has failed.
int keep_running(gpuos_ctx* c, bool query_stream) {
  if (c->host_only || c->exited || c->parked) return 0;
  bool gone = load_acq(&c->hctl->exit_epoch) == c->epoch;
  if (!gone && load_acq(&c->hctl->exit_req) == c->epoch) {
    // the doorbell is deciding whether to leave: it either completes the exit
    // or withdraws the announcement within microseconds
    const auto t0 = std::chrono::steady_clock::now();
    for (;;) {
      gone = load_acq(&c->hctl->exit_epoch) == c->epoch;
      if (gone || load_acq(&c->hctl->exit_req) != c->epoch) break;
      if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(10)) {
        c->poisoned = true;
        return fail(GPUOS_EDEVICE, "resident kernel neither left nor resumed");
      }
      cpu_relax();
    }
  }
  if (!gone && query_stream) {
    const hipError_t e = hipStreamQuery(c->stream);
    if (e == hipErrorNotReady) return 0;
    // the exit announcement precedes the end of the launch
    gone = load_acq(&c->hctl->exit_epoch) == c->epoch;
    if (!gone || e != hipSuccess) {
      c->poisoned = true;
      c->exited = true;
      return fail(GPUOS_EDEVICE, "resident kernel is no longer running: %s", hipGetErrorString(e));
    }
  }
  if (!gone) return 0;
  int rc = wait_kernel_end(c, 10ll * 1000 * 1000 * 1000);
  if (rc) return rc;
  account_launch(c);
  if (c->stopped) {
    c->exited = true;
    return 0;
  }
  return launch_kernel(c, load_acq(&c->hctl->exit_tiles));
}

// Waits until ring slot for `seq` is free; returns 0, EAGAIN or EDEVICE.
int wait_ring_space(gpuos_ctx* c, uint32_t ring, uint64_t seq) {
  if (seq <= (uint64_t)c->cap || seq - c->cap <= completed_of(c, ring)) return 0;
  if ((c->host_only && !c->consumer) || c->cfg.block_on_full == 2)
    return fail(GPUOS_EAGAIN, "ring %u full (%u slots)", ring, c->cap);
  ++c->st.ring_full_waits;
  // make what is already written visible so the device can drain it
  if (c->tail_written[ring] != c->pub_seq[ring]) {
    store_rel(&c->hctl->tail[ring], c->pub_seq[ring]);
    if (ring == 1) store_rel(&c->hctl->lc_tail, c->pub_seq[1]);
    c->tail_written[ring] = c->pub_seq[ring];
  }
  uint32_t spins = 0;
  const auto t0 = std::chrono::steady_clock::now();
  while (seq - c->cap > completed_of(c, ring)) {
    if (check_device_error(c)) return GPUOS_EDEVICE;
    if (c->host_only && std::chrono::steady_clock::now() - t0 > std::chrono::seconds(30))
      return fail(GPUOS_ETIMEDOUT, "ring %u full: the consumer retired nothing for 30 s", ring);
    if (++spins > 256) {
      std::this_thread::yield();
      if ((spins & 1023) == 0) {
        const int rc = keep_running(c, (spins & 0xffff) == 0);
        if (rc) return rc;
      }
    } else {
      cpu_relax();
    }
  }
  return 0;
}

void publish_tail(gpuos_ctx* c, uint32_t ring) {
  if (c->tail_written[ring] == c->pub_seq[ring]) return;
  std::atomic_thread_fence(std::memory_order_release);
  store_rel(&c->hctl->tail[ring], c->pub_seq[ring]);
  if (ring == 1) store_rel(&c->hctl->lc_tail, c->pub_seq[1]);
  c->tail_written[ring] = c->pub_seq[ring];
}

// Writes one planned descriptor into its ring and records the id -> seq map.
int publish_one(gpuos_ctx* c, Planned& pl) {
  const uint32_t ring = pl.ring;
  const uint64_t seq = c->pub_seq[ring] + 1;
  int rc = wait_ring_space(c, ring, seq);
  if (rc) return rc;
  DevDesc& d = pl.desc;
  d.seq = seq;
  d.check = (uint32_t)seq ^ kDescMagic;
  d.tstart = c->pub_tiles[ring];
  // dependencies -> sequences of the same ring; drop completed ones
  DepVec dseq;
  for (uint64_t dep : pl.deps) {
    if (id_retired(c, dep)) continue;
    const uint64_t v = c->idseq[dep - c->id_base];
    const uint32_t dring = (uint32_t)(v >> 63);
    const uint64_t s = v & ((1ull << 63) - 1);
    if (dring != ring) {
      // a dependency across rings is honoured on the host: wait for it
      publish_tail(c, dring);
      publish_tail(c, ring);
      uint32_t spins = 0;
      while (s > completed_of(c, dring)) {
        if (check_device_error(c)) return GPUOS_EDEVICE;
        if (c->host_only && !c->consumer) return fail(GPUOS_EAGAIN, "cross-ring dependency pending");
        if ((++spins & 1023) == 0) {
          const int rc2 = keep_running(c, (spins & 0xffff) == 0);
          if (rc2) return rc2;
        }
        std::this_thread::yield();
      }
      continue;
    }
    dseq.push_back(s);
  }
  dseq.sort_unique();
  // Dependencies implied by another are dropped, so waves poll fewer
  // completion words.  A descriptor's prefix k says that descriptors 1..k of
  // its ring have all completed whenever it starts: those the host saw
  // retired before publishing it, its dependencies and, through them, theirs.
  // A dependency at or below another dependency's prefix completed before
  // that one started, so waiting for the latter covers it: its stores were
  // acknowledged before its completion was counted.
  std::vector<uint64_t>& prefix = c->done_prefix[ring];
  uint64_t pre = completed_of(c, ring);
  for (uint64_t s : dseq) pre = std::max(pre, prefix[(s - 1) & (c->cap - 1)]);
  dseq.remove_if([pre](uint64_t s) { return s <= pre; });
  for (uint64_t s : dseq)
    if (s == pre + 1) pre = s;  // ascending: consecutive dependencies extend it
  if (dseq.size() <= (size_t)kMaxDeps) {
    // seq - dep fits 32 bits: a live dependency is less than a ring behind
    for (size_t k = 0; k < dseq.size(); ++k) {
      const uint32_t delta = (uint32_t)(seq - dseq[k]);
      if (k < 8)
        d.deps_lo[k] = delta;
      else
        d.deps_hi[k - 8] = delta;
    }
  } else {
    d.wait_retired = dseq.back();  // retire order covers every dependency
    pre = dseq.back();
  }
  prefix[(seq - 1) & (c->cap - 1)] = pre;
  DevDesc* slot = &c->hdesc[ring][(seq - 1) & (c->cap - 1)];
  memcpy(slot, &d, sizeof d);
  c->hends[ring][(seq - 1) & (c->cap - 1)] = c->pub_tiles[ring] + d.ntiles;
  c->pub_tiles[ring] += d.ntiles;
  c->pub_seq[ring] = seq;
  for (uint32_t k = 0; k < pl.count; ++k) {
    const uint64_t id = c->staged[pl.first + k].id;
    c->idseq[id - c->id_base] = ((uint64_t)ring << 63) | seq;
  }
  ++c->st.descs_published;
  if ((seq & 63) == 0) publish_tail(c, ring);
  return 0;
}

// Can the compiled kernel variant run descriptor d?  (Its op table: PROGRAM
// ops with a compiled body, NOP, 4-byte COPY, fp32 elementwise ops and fused
// fp32 chains, no views.)
bool rtc_runnable(const DevDesc& d) {
  if (d.flags & DF_VIEW) return false;
  switch (d.opcode) {
    case GPUOS_OP_PROGRAM:
      return d.pg.body != 0;
    case GPUOS_OP_NOP:
      return true;
    case GPUOS_OP_COPY:
      return d.dtype == GPUOS_F32 || d.dtype == GPUOS_I32;
    case GPUOS_OP_ADD: case GPUOS_OP_MUL: case GPUOS_OP_RELU: case GPUOS_OP_SCALE:
    case GPUOS_OP_EXP: case GPUOS_OP_SILU_MUL: case OP_FUSED_EW:
      return d.dtype == GPUOS_F32;
    default:
      return false;
  }
}

// The resident kernel leaves once the queue is drained (the doorbell wave
// runs the same exit handshake as an idle exit; it may also have idled out
// already) and the context is parked: the next launch starts at park_tiles.
int park_kernel(gpuos_ctx* c, int64_t timeout_ns) {
  std::atomic_thread_fence(std::memory_order_seq_cst);
  store_rel(&c->hctl->yield_req, 1);
  const auto t0 = std::chrono::steady_clock::now();
  while (load_acq(&c->hctl->exit_epoch) != c->epoch) {
    if (check_device_error(c)) {
      store_rel(&c->hctl->yield_req, 0);
      return GPUOS_EDEVICE;
    }
    if (timeout_ns >= 0 &&
        std::chrono::steady_clock::now() - t0 > std::chrono::nanoseconds(timeout_ns)) {
      store_rel(&c->hctl->yield_req, 0);
      return fail(GPUOS_ETIMEDOUT, "the resident kernel did not leave");
    }
    std::this_thread::sleep_for(std::chrono::microseconds(2));
  }
  store_rel(&c->hctl->yield_req, 0);
  const int rc = wait_kernel_end(c, timeout_ns);
  if (rc) return rc;
  account_launch(c);
  c->park_tiles = load_acq(&c->hctl->exit_tiles);
  c->parked = true;
  return 0;
}

// Hands the queue to the compiled variant rtc_new (to_rtc) or to the
// built-in kernel, at a drain point: every published op completes, the
// running kernel leaves, and the other kernel is launched on the same rings
// from the ticket where the first one stopped.  The variant the previous
// kernel ran is released here unless it is also the latest compile.
constexpr int64_t kSwitchTimeoutNs = 60ll * 1000 * 1000 * 1000;
int sync_impl(gpuos_ctx* c, uint64_t upto, int64_t timeout_ns);

int switch_kernel(gpuos_ctx* c, bool to_rtc) {
  ++c->st.kernel_switches;
  if (c->host_only) {  // nothing runs: the hand-over is only counted
    c->on_rtc = to_rtc;
    c->rtc_run = to_rtc ? c->rtc_new : nullptr;
    return 0;
  }
  if (!c->parked) {
    int rc = sync_impl(c, 0, kSwitchTimeoutNs);
    if (!rc) rc = park_kernel(c, kSwitchTimeoutNs);
    if (rc) return rc;
  }
  c->on_rtc = to_rtc;
  c->rtc_run = to_rtc ? c->rtc_new : nullptr;
  const int rc = launch_kernel(c, c->park_tiles);
  if (!rc) c->parked = false;
  return rc;
}

int flush_impl(gpuos_ctx* c) {
  if (check_device_error(c)) return GPUOS_EDEVICE;
  if (c->staged.empty()) return 0;
  ++c->st.flushes;
  std::vector<Planned>& plan = c->plan;
  plan.clear();
  plan.reserve(c->staged.size());
  plan_ops(c, 0, c->staged.size(), plan);
  // Kernel hand-overs: to the compiled variant before a PROGRAM op with a
  // compiled body if it can run every descriptor left in this flush; back to
  // the built-in kernel before one it cannot run; from an older variant to
  // the latest before a body only the latest holds.
  const bool variants = c->rtc_new || c->on_rtc;
  std::vector<uint8_t>& tail_ok = c->tail_ok;
  if (variants) {
    tail_ok.assign(plan.size() + 1, 1);
    for (size_t i = plan.size(); i-- > 0;) tail_ok[i] = tail_ok[i + 1] && rtc_runnable(plan[i].desc);
  }
  auto wanted = [&](size_t i) -> int {  // -1 = stay, 0 = built-in, 1 = latest variant
    const DevDesc& d = plan[i].desc;
    const bool compiled = d.opcode == GPUOS_OP_PROGRAM && d.pg.body != 0;
    if (c->on_rtc) {
      if (!rtc_runnable(d)) return 0;
      return compiled && c->rtc_run != c->rtc_new ? 1 : -1;
    }
    return compiled && tail_ok[i] ? 1 : -1;
  };
  int rc = 0;
  if (c->parked) {  // relaunch first: publication may wait for ring space
    if (variants && !plan.empty()) {
      const int w = wanted(0);
      if (w >= 0) {
        ++c->st.kernel_switches;
        c->on_rtc = w == 1;
        c->rtc_run = c->on_rtc ? c->rtc_new : nullptr;
      }
    }
    rc = launch_kernel(c, c->park_tiles);
    if (rc) return rc;
    c->parked = false;
  }
  size_t done_ops = 0;
  for (size_t i = 0; i < plan.size(); ++i) {
    Planned& pl = plan[i];
    if (variants) {
      const int w = wanted(i);
      if (w >= 0) {
        publish_tail(c, 0);
        publish_tail(c, 1);
        rc = switch_kernel(c, w == 1);
        if (rc) break;
      }
    }
    rc = publish_one(c, pl);
    if (rc) break;
    if (pl.desc.opcode == GPUOS_OP_PROGRAM && pl.desc.pg.body) ++c->st.programs_compiled;
    done_ops += pl.count;
  }
  publish_tail(c, 0);
  publish_tail(c, 1);
  c->staged.erase(c->staged.begin(), c->staged.begin() + done_ops);
  // the tail stores above come before the look at the exit announcement
  std::atomic_thread_fence(std::memory_order_seq_cst);
  if (!rc) rc = keep_running(c, false);
  return rc;
}

int alloc_host(gpuos_ctx* c, void** p, size_t bytes) {
  if (c->host_only) {
    *p = aligned_alloc(256, (bytes + 255) / 256 * 256);
    if (!*p) return fail(GPUOS_ENOMEM, "host allocation of %zu bytes failed", bytes);
    memset(*p, 0, bytes);
    return 0;
  }
  hipError_t e = hipHostMalloc(p, bytes, hipHostMallocCoherent | hipHostMallocMapped);
  if (e != hipSuccess) return fail(GPUOS_ENOMEM, "hipHostMalloc(%zu): %s", bytes, hipGetErrorString(e));
  memset(*p, 0, bytes);
  return 0;
}

void free_host(gpuos_ctx* c, void* p) {
  if (!p) return;
  if (c->host_only)
    free(p);
  else
    (void)hipHostFree(p);
}

// One static-scratch context per device at a time (they share the array).
std::atomic<bool> g_static_busy[kMaxStaticDevices];

void free_all(gpuos_ctx* c) {
  if (c->static_mem) {
    // the rings live in the caller's workspace and the static scratch
    if (c->ev_start) (void)hipEventDestroy(c->ev_start);
    if (c->ev_end) (void)hipEventDestroy(c->ev_end);
    if (c->stream) (void)hipStreamDestroy(c->stream);
    g_static_busy[c->device].store(false, std::memory_order_release);
    return;
  }
  free_host(c, c->hctl);
  free_host(c, c->hdone_lc);
  for (int r = 0; r < kRings; ++r) {
    free_host(c, c->hdesc[r]);
    free_host(c, c->hends[r]);
  }
  if (!c->host_only) {
    (void)hipFree(c->dctl);
    for (int r = 0; r < kRings; ++r) {
      (void)hipFree(c->ddesc[r]);
      (void)hipFree(c->dends[r]);
      (void)hipFree(c->done_id[r]);
      (void)hipFree(c->tiles_done[r]);
      (void)hipFree(c->subs_done[r]);
      (void)hipFree(c->trace[r]);
      (void)hipFree(c->tile_exec[r]);
    }
    if (c->ev_start) (void)hipEventDestroy(c->ev_start);
    if (c->ev_end) (void)hipEventDestroy(c->ev_end);
    if (c->stream) (void)hipStreamDestroy(c->stream);
  }
}

void* dev_ptr(void* host) {
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, host, 0) != hipSuccess) return host;
  return d;
}

// Environment overrides of the defaults: GPUOS_<FIELD> (the field's name in
// capitals, a decimal or 0x-prefixed value) replaces the default of that
// field; a nonzero field in the caller's config still wins.  A malformed
// value is an error, so that a typo is not silently ignored.
int env_defaults(gpuos_config& out) {
  struct F { const char* name; uint32_t* field; };
  const F fields[] = {
      {"GPUOS_RING_SLOTS", &out.ring_slots}, {"GPUOS_WAVES_PER_CU", &out.waves_per_cu},
      {"GPUOS_TILE_ELEMS", &out.tile_elems}, {"GPUOS_BE_TILE_ELEMS", &out.be_tile_elems},
      {"GPUOS_FUSION", &out.fusion}, {"GPUOS_AUTO_DEPS", &out.auto_deps}, {"GPUOS_TRACE", &out.trace},
      {"GPUOS_BLOCK_ON_FULL", &out.block_on_full}, {"GPUOS_MAX_FUSE", &out.max_fuse},
      {"GPUOS_PRIORITY", &out.priority}, {"GPUOS_IDLE_EXIT_MS", &out.idle_exit_ms},
      {"GPUOS_STREAM_MIN_KIB", &out.stream_min_kib}, {"GPUOS_LC_WAVES", &out.lc_waves},
      {"GPUOS_TILE_COUNTS", &out.tile_counts}, {"GPUOS_JITTER", &out.jitter}};
  for (const F& f : fields) {
    const char* v = getenv(f.name);
    if (!v || !*v) continue;
    char* end = nullptr;
    const unsigned long long x = strtoull(v, &end, 0);
    if (*end || x > 0xFFFFFFFFull) return fail(GPUOS_EINVAL, "%s=%s is not a 32-bit unsigned number", f.name, v);
    *f.field = (uint32_t)x;
  }
  return 0;
}

int apply_config(const gpuos_config* in, gpuos_config& out) {
  gpuos_config_default(&out);
  if (int rc = env_defaults(out)) return rc;
  if (in) {
    if (in->ring_slots) out.ring_slots = in->ring_slots;
    if (in->waves_per_cu) out.waves_per_cu = in->waves_per_cu;
    if (in->tile_elems) out.tile_elems = in->tile_elems;
    if (in->be_tile_elems) out.be_tile_elems = in->be_tile_elems;
    if (in->fusion) out.fusion = in->fusion;
    if (in->auto_deps) out.auto_deps = in->auto_deps;
    if (in->trace) out.trace = in->trace;
    if (in->block_on_full) out.block_on_full = in->block_on_full;
    if (in->max_fuse) out.max_fuse = in->max_fuse;
    if (in->priority) out.priority = in->priority;
    if (in->idle_exit_ms) out.idle_exit_ms = in->idle_exit_ms;
    if (in->stream_min_kib) out.stream_min_kib = in->stream_min_kib;
    if (in->lc_waves) out.lc_waves = in->lc_waves;
    if (in->tile_counts) out.tile_counts = in->tile_counts;
    if (in->jitter) out.jitter = in->jitter;
    if (in->reserved) return fail(GPUOS_EINVAL, "reserved config field must be 0");
  }
  if (out.jitter > 1000) return fail(GPUOS_EINVAL, "jitter must be at most 1000");
  const uint32_t rs = out.ring_slots;
  if (rs < 64 || rs > (1u << 18) || (rs & (rs - 1)))
    return fail(GPUOS_EINVAL, "ring_slots must be a power of two in [64, 2^18]");
  if (out.waves_per_cu < 4 || out.waves_per_cu > 32 || out.waves_per_cu % 4)
    return fail(GPUOS_EINVAL, "waves_per_cu must be a multiple of 4 in [4, 32]");
  if (out.tile_elems < 256 || out.tile_elems % 256 || out.tile_elems > (1u << 22))
    return fail(GPUOS_EINVAL, "tile_elems must be a multiple of 256 in [256, 2^22]");
  if (out.be_tile_elems < 256 || out.be_tile_elems % 256 || out.be_tile_elems > (1u << 22))
    return fail(GPUOS_EINVAL, "be_tile_elems must be a multiple of 256 in [256, 2^22]");
  if (out.fusion > 2 || out.auto_deps > 2 || out.trace > 2 || out.block_on_full > 2 ||
      out.priority > 2)
    return fail(GPUOS_EINVAL, "switch fields take 1 (on) or 2 (off)");
  if (out.lc_waves < 1 || out.lc_waves > 64)
    return fail(GPUOS_EINVAL, "lc_waves must be in [1, 64]");
  if (out.max_fuse < 2 || out.max_fuse > (uint32_t)kMaxSteps)
    return fail(GPUOS_EINVAL, "max_fuse must be in [2, 8]");
  return 0;
}

int sync_impl(gpuos_ctx* c, uint64_t upto, int64_t timeout_ns) {
  uint64_t target[kRings] = {c->pub_seq[0], c->pub_seq[1]};
  if (upto) {
    if (upto >= c->next_id) return fail(GPUOS_EINVAL, "sync: id %llu was never submitted",
                                        (unsigned long long)upto);
    target[0] = target[1] = 0;
    bool found[kRings] = {false, false};
    for (uint64_t id = upto; id >= c->id_base && !(found[0] && found[1]); --id) {
      const uint64_t v = c->idseq[id - c->id_base];
      const uint32_t r = (uint32_t)(v >> 63);
      if (!found[r]) {
        target[r] = v & ((1ull << 63) - 1);
        found[r] = true;
      }
      if (id == c->id_base) break;
    }
  }
  const auto t0 = std::chrono::steady_clock::now();
  uint32_t spins = 0;
  for (int r = 0; r < kRings; ++r) {
    while (completed_of(c, r) < target[r]) {
      if (check_device_error(c)) return GPUOS_EDEVICE;
      if (c->host_only && !c->consumer)
        return fail(GPUOS_ETIMEDOUT, "host-only context: ops never complete");
      ++spins;
      if (spins < 2048) {
        cpu_relax();
        continue;
      }
      if ((spins & 1023) == 0) {
        if (timeout_ns >= 0) {
          const auto el = std::chrono::duration_cast<std::chrono::nanoseconds>(
                              std::chrono::steady_clock::now() - t0)
                              .count();
          if (el > timeout_ns)
            return fail(GPUOS_ETIMEDOUT, "sync timed out: ring %d at %llu of %llu", r,
                        (unsigned long long)completed_of(c, r), (unsigned long long)target[r]);
        }
        const int rc = keep_running(c, (spins & 0xffff) == 0);
        if (rc) return rc;
      }
      std::this_thread::yield();
    }
  }
  if (check_device_error(c)) return GPUOS_EDEVICE;
  prune_ids(c);
  return 0;
}

// ---------------------------------------------------------------------------
// compiled kernel variant (gpuos_program_compile)

// Source register r of a body: r0..r7 are variables, r8..r15 the program's
// constants, written as their exact bits.
std::string rtc_reg(const ProgCode& pc, uint32_t r) {
  if (r < 8) return "r" + std::to_string(r);
  uint32_t bits;
  memcpy(&bits, &pc.k[r - 8], 4);
  char buf[64];
  snprintf(buf, sizeof buf, "pvec(__uint_as_float(0x%08xu))", bits);
  return buf;
}

// Program pc as straight-line code: a functor over 4-element vectors with
// one statement per instruction, each the interpreter's operation for it
// (the pv_* helpers are the interpreter's own).  r0..r2 arrive as the
// inputs (+0 past n_inputs); r3..r7 start at +0, as registers the program
// reads before writing do in the interpreter.
void emit_body(std::string& s, uint32_t k, const ProgCode& pc) {
  s += "struct RtcBody" + std::to_string(k) + " {\n";
  s += "  __device__ __forceinline__ pvec operator()(pvec r0, pvec r1, pvec r2) const {\n";
  s += "    [[maybe_unused]] pvec r3 = pvec(0.0f), r4 = r3, r5 = r3, r6 = r3, r7 = r3;\n";
  const uint32_t ni = pc.meta & 31u;
  for (uint32_t i = 0; i < ni; ++i) {
    const uint32_t w = pc.ins[i];
    const uint32_t op = w & 31u, dst = (w >> 5) & 7u;
    const std::string a = rtc_reg(pc, (w >> 8) & 15u), b = rtc_reg(pc, (w >> 12) & 15u),
                      cc = rtc_reg(pc, (w >> 16) & 15u);
    std::string e;
    switch (op) {
      case GPUOS_P_ADD: e = a + " + " + b; break;
      case GPUOS_P_SUB: e = a + " - " + b; break;
      case GPUOS_P_MUL: e = a + " * " + b; break;
      case GPUOS_P_DIV: e = a + " / " + b; break;
      case GPUOS_P_MIN: e = "pv_min(" + a + ", " + b + ")"; break;
      case GPUOS_P_MAX: e = "pv_max(" + a + ", " + b + ")"; break;
      case GPUOS_P_NEG: e = "pv_neg(" + a + ")"; break;
      case GPUOS_P_ABS: e = "pv_abs(" + a + ")"; break;
      case GPUOS_P_RELU: e = "pv_relu(" + a + ")"; break;
      case GPUOS_P_EXP: e = "pv_exp(" + a + ")"; break;
      case GPUOS_P_LT: e = "pv_lt(" + a + ", " + b + ")"; break;
      case GPUOS_P_SEL: e = "pv_sel(" + a + ", " + b + ", " + cc + ")"; break;
      default: e = a; break;  // MOV
    }
    s += "    r" + std::to_string(dst) + " = " + e + ";\n";
  }
  s += "    return " + rtc_reg(pc, (pc.meta >> 8) & 15u) + ";\n  }\n};\n";
}

const char kRtcMain[] = "#define GPUOS_RTC_VARIANT 1\n#include \"kernels.hip\"\n";
// hipRTC has no hip/hip_runtime.h (its device API is built in) and no
// stddef.h: these stand in for them.
const char kRtcHipRuntime[] = "#pragma once\n";
const char kRtcStddef[] =
    "#pragma once\ntypedef decltype(sizeof(0)) size_t;\n#define offsetof(t, m) __builtin_offsetof(t, m)\n";

// Compiles the variant with `bodies` as gpuos_rtc_bodies.h for target
// `arch`; the code object goes to `code`, the compiler's messages to `log`.
int rtc_compile(const std::string& arch, const std::string& bodies, std::vector<char>& code,
                std::string& log) {
  std::vector<const char*> names, texts;
  for (unsigned i = 0; i < kRtcSourceCount; ++i) {
    names.push_back(kRtcSourceNames[i]);
    texts.push_back(kRtcSourceTexts[i]);
  }
  names.push_back("hip/hip_runtime.h");
  texts.push_back(kRtcHipRuntime);
  names.push_back("stddef.h");
  texts.push_back(kRtcStddef);
  names.push_back("gpuos_rtc_bodies.h");
  texts.push_back(bodies.c_str());
  hiprtcProgram prog;
  hiprtcResult r = hiprtcCreateProgram(&prog, kRtcMain, "gpuos_resident_rtc.hip", (int)names.size(),
                                       texts.data(), names.data());
  if (r != HIPRTC_SUCCESS) return fail(GPUOS_ECOMPILE, "hiprtcCreateProgram: %s", hiprtcGetErrorString(r));
  // the flags the library's own kernels are built with
  const std::string target = "--offload-arch=" + arch;
  const char* opts[] = {target.c_str(), "-O3", "-std=c++17", "-ffp-contract=off",
                        "-fno-gpu-flush-denormals-to-zero", "-Xclang", "-target-feature", "-Xclang",
                        "-packed-fp32-ops"};
  r = hiprtcCompileProgram(prog, (int)(sizeof opts / sizeof opts[0]), opts);
  size_t n = 0;
  if (hiprtcGetProgramLogSize(prog, &n) == HIPRTC_SUCCESS && n > 1) {
    log.assign(n, '\0');
    if (hiprtcGetProgramLog(prog, &log[0]) != HIPRTC_SUCCESS) log.clear();
    while (!log.empty() && log.back() == '\0') log.pop_back();
  }
  if (r == HIPRTC_SUCCESS) {
    n = 0;
    r = hiprtcGetCodeSize(prog, &n);
    if (r == HIPRTC_SUCCESS && n) {
      code.resize(n);
      r = hiprtcGetCode(prog, code.data());
    }
  }
  (void)hiprtcDestroyProgram(&prog);
  if (r != HIPRTC_SUCCESS || code.empty())
    return fail(GPUOS_ECOMPILE, "hipRTC compile failed: %s", hiprtcGetErrorString(r));
  return 0;
}

// Loads a compiled variant and checks that it fits the context's resident
// grid (the built-in kernel's blocks per CU) without scratch memory.
int rtc_load(gpuos_ctx* c, const std::vector<char>& code, RtcModule& m) {
  HIP_TRY(hipSetDevice(c->device));
  HIP_TRY(hipModuleLoadData(&m.mod, code.data()));
  HIP_TRY(hipModuleGetFunction(&m.fn, m.mod, "gpuos_resident_rtc"));
  int scratch = 0, nb = 0;
  HIP_TRY(hipFuncGetAttribute(&scratch, HIP_FUNC_ATTRIBUTE_LOCAL_SIZE_BYTES, m.fn));
  HIP_TRY(hipModuleOccupancyMaxActiveBlocksPerMultiprocessor(&nb, m.fn, 256, 0));
  const uint32_t bpc = c->blocks / c->cus;
  if (scratch != 0 || (uint32_t)nb < bpc)
    return fail(GPUOS_ECOMPILE, "compiled variant fits %d blocks per CU (%u needed) and uses %d B of scratch",
                nb, bpc, scratch);
  return 0;
}

// Memory a static context is built in (gpuos_create_static).
struct StaticMem {
  void* host;                // the caller's pinned workspace (host address)
  void* dev;                 // the device's static scratch
  bool handed_over = false;  // the context now owns the device's busy flag
};

int create_impl(int device, const gpuos_config* cfg_in, StaticMem* sm, gpuos_ctx** out);

}  // namespace

// ===========================================================================
// C ABI

extern "C" {

int gpuos_abi_version(void) { return GPUOS_ABI_VERSION; }

const char* gpuos_last_error(void) { return g_last_error.c_str(); }

void gpuos_config_default(gpuos_config* cfg) {
  if (!cfg) return;
  memset(cfg, 0, sizeof *cfg);
  cfg->ring_slots = 65536;
  cfg->waves_per_cu = 8;
  cfg->tile_elems = 1024;
  cfg->be_tile_elems = 32768;
  cfg->fusion = 1;
  cfg->auto_deps = 1;
  cfg->trace = 2;
  cfg->block_on_full = 1;
  cfg->max_fuse = 8;
  cfg->priority = 1;
  cfg->idle_exit_ms = 200;
  cfg->stream_min_kib = 32768;
  cfg->lc_waves = 8;
}

int gpuos_create(int device, const gpuos_config* cfg_in, gpuos_ctx** out) {
  return create_impl(device, cfg_in, nullptr, out);
}

int gpuos_create_static(int device, const gpuos_config* cfg_in, void* host_ws, size_t host_ws_bytes,
                        gpuos_ctx** out) {
  if (!out) return fail(GPUOS_EINVAL, "out is null");
  *out = nullptr;
  gpuos_config cfg;
  int rc = apply_config(cfg_in, cfg);
  if (rc) return rc;
  if (device < 0 || device >= kMaxStaticDevices)
    return fail(GPUOS_EINVAL, "device %d: static contexts exist for devices 0..%d", device,
                kMaxStaticDevices - 1);
  if (cfg.ring_slots > kStaticMaxSlots)
    return fail(GPUOS_EINVAL, "ring_slots %u: a static context holds at most %u slots per ring "
                "(%zu bytes of static device scratch)", cfg.ring_slots, kStaticMaxSlots,
                kStaticScratchBytes);
  if (cfg.trace == 1 || cfg.tile_counts)
    return fail(GPUOS_EINVAL, "trace and tile_counts need allocations: not available in a static context");
  const size_t need = static_host_bytes(cfg.ring_slots);
  if (!host_ws || ((uintptr_t)host_ws & 255) || host_ws_bytes < need)
    return fail(GPUOS_EINVAL, "host workspace: need %zu bytes, 256-byte aligned (got %zu at %p)", need,
                host_ws_bytes, host_ws);
  unsigned int flags = 0;
  if (hipHostGetFlags(&flags, host_ws) != hipSuccess ||
      (flags & (hipHostMallocMapped | hipHostMallocCoherent)) != (hipHostMallocMapped | hipHostMallocCoherent))
    return fail(GPUOS_EINVAL, "host workspace must come from hipHostMalloc with hipHostMallocMapped | "
                "hipHostMallocCoherent (flags %#x)", flags);
  bool expect = false;
  if (!g_static_busy[device].compare_exchange_strong(expect, true, std::memory_order_acq_rel))
    return fail(GPUOS_ESTATE, "device %d already has a live static context: contexts on one device "
                "share its static scratch", device);
  void* dev = nullptr;
  const hipError_t e = static_scratch(device, &dev);
  if (e != hipSuccess || !dev) {
    g_static_busy[device].store(false, std::memory_order_release);
    return fail(GPUOS_EDEVICE, "static scratch of device %d: %s", device, hipGetErrorString(e));
  }
  StaticMem sm{host_ws, dev};
  rc = create_impl(device, &cfg, &sm, out);
  if (rc && !*out && !sm.handed_over) g_static_busy[device].store(false, std::memory_order_release);
  return rc;
}

}  // extern "C"

namespace {

int create_impl(int device, const gpuos_config* cfg_in, StaticMem* sm, gpuos_ctx** out) {
  if (!out) return fail(GPUOS_EINVAL, "out is null");
  *out = nullptr;
  gpuos_config cfg;
  int rc = apply_config(cfg_in, cfg);
  if (rc) return rc;
  auto* c = new gpuos_ctx();
  c->cfg = cfg;
  c->cap = cfg.ring_slots;
  for (int r = 0; r < kRings; ++r) c->done_prefix[r].assign(c->cap, 0);
  c->device = device;
  c->host_only = device == GPUOS_DEVICE_NONE;
  if (!c->host_only) {
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev) {
      delete c;
      return fail(GPUOS_EINVAL, "no HIP device %d (%d visible)", device, ndev);
    }
    hipError_t e = hipSetDevice(device);
    hipDeviceProp_t prop;
    if (e == hipSuccess) e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) {
      delete c;
      return fail(GPUOS_EDEVICE, "device %d: %s", device, hipGetErrorString(e));
    }
    c->cus = (uint32_t)prop.multiProcessorCount;
    c->arch = prop.gcnArchName;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, resident_kernel(), 256, 0);
    if (e != hipSuccess || nb <= 0) {
      delete c;
      return fail(GPUOS_EDEVICE, "occupancy query failed: %s", hipGetErrorString(e));
    }
    uint32_t bpc = cfg.waves_per_cu / 4;
    if (bpc > (uint32_t)nb) {
      delete c;
      return fail(GPUOS_EINVAL, "waves_per_cu %u exceeds the kernel's occupancy (%d blocks of 4 waves)",
                  cfg.waves_per_cu, nb);
    }
    c->blocks = c->cus * bpc;
  } else {
    c->cus = 256;
    c->blocks = c->cus * (cfg.waves_per_cu / 4);
  }
  c->lc_waves = cfg.priority == 1 ? cfg.lc_waves : 0;
  if (c->lc_waves + 64 > c->blocks * 4) {
    delete c;
    return fail(GPUOS_EINVAL, "lc_waves %u leaves too few best-effort waves", cfg.lc_waves);
  }
  c->workers = c->blocks * 4 - 1 - c->lc_waves;
  c->st.worker_waves = c->workers;
  c->st.lc_waves = c->lc_waves;
  c->st.compute_units = c->cus;

  if (sm) {
    // carve the caller's pinned workspace and the static device scratch in
    // the order static_host_bytes / static_device_bytes count them
    c->static_mem = true;
    sm->handed_over = true;  // from here on free_all releases the device
    uint8_t* h = static_cast<uint8_t*>(sm->host);
    memset(h, 0, static_host_bytes(c->cap));
    c->hctl = reinterpret_cast<HostCtl*>(h);
    h += align256(sizeof(HostCtl));
    for (int r = 0; r < kRings; ++r) {
      c->hdesc[r] = reinterpret_cast<DevDesc*>(h);
      h += align256((size_t)c->cap * kDescBytes);
      c->hends[r] = reinterpret_cast<uint64_t*>(h);
      h += align256((size_t)c->cap * 8);
    }
    c->hdone_lc = reinterpret_cast<uint64_t*>(h);
  } else {
    rc = alloc_host(c, (void**)&c->hctl, sizeof(HostCtl));
    for (int r = 0; r < kRings && !rc; ++r) {
      rc = alloc_host(c, (void**)&c->hdesc[r], (size_t)c->cap * sizeof(DevDesc));
      if (!rc) rc = alloc_host(c, (void**)&c->hends[r], (size_t)c->cap * sizeof(uint64_t));
    }
    if (!rc) rc = alloc_host(c, (void**)&c->hdone_lc, (size_t)c->cap * sizeof(uint64_t));
  }
  if (rc) {
    free_all(c);
    delete c;
    return rc;
  }
  if (!c->host_only) {
    uint8_t* carve = sm ? static_cast<uint8_t*>(sm->dev) : nullptr;
    auto dalloc = [&](void** p, size_t bytes) -> int {
      if (carve) {  // static scratch: consecutive 256-byte aligned pieces
        *p = carve;
        carve += align256(bytes);
        return 0;
      }
      hipError_t e = hipMalloc(p, bytes);
      if (e != hipSuccess) return fail(GPUOS_ENOMEM, "hipMalloc(%zu): %s", bytes, hipGetErrorString(e));
      return 0;
    };
    rc = dalloc((void**)&c->dctl, sizeof(DevCtl));
    for (int r = 0; r < kRings && !rc; ++r) {
      rc = dalloc((void**)&c->ddesc[r], (size_t)c->cap * sizeof(DevDesc));
      if (!rc) rc = dalloc((void**)&c->dends[r], (size_t)2 * c->cap * sizeof(uint64_t));
      if (!rc) rc = dalloc((void**)&c->done_id[r], (size_t)c->cap * kDoneReplicas * sizeof(uint64_t));
      if (!rc) rc = dalloc((void**)&c->tiles_done[r], (size_t)kSubCounters * c->cap * sizeof(uint32_t));
      if (!rc) rc = dalloc((void**)&c->subs_done[r], (size_t)c->cap * sizeof(uint32_t));
      if (!rc && cfg.trace == 1) rc = dalloc((void**)&c->trace[r], (size_t)c->cap * sizeof(TraceRec));
      if (!rc && cfg.tile_counts) rc = dalloc((void**)&c->tile_exec[r], (size_t)cfg.tile_counts * 4);
    }
    hipError_t e = hipSuccess;
    if (!rc) e = hipStreamCreateWithFlags(&c->stream, hipStreamNonBlocking);
    if (!rc && e == hipSuccess) {
      // control block: zeros, except that no wave may stop yet
      static_assert(sizeof(DevCtl) <= 16384, "control block image fits the stack");
      DevCtl img_storage;
      DevCtl* img = &img_storage;
      memset(img, 0, sizeof *img);
      for (int r = 0; r < kRings; ++r)
        for (uint32_t k = 0; k < kReplicas; ++k) img->avail[r][k].stop_ticket = ~0ull;  // epoch 0
      for (int r = 0; r < kRings; ++r) img->tile_exec[r] = c->tile_exec[r];
      img->tile_exec_n = cfg.tile_counts;
      img->hdone_lc = (uint64_t*)dev_ptr(c->hdone_lc);
      e = hipMemcpy(c->dctl, img, sizeof(DevCtl), hipMemcpyHostToDevice);
      for (int r = 0; r < kRings && e == hipSuccess; ++r) {
        e = hipMemsetAsync(c->dends[r], 0, (size_t)2 * c->cap * sizeof(uint64_t), c->stream);
        if (e == hipSuccess) e = hipMemsetAsync(c->ddesc[r], 0, (size_t)c->cap * sizeof(DevDesc), c->stream);
        if (e == hipSuccess)
          e = hipMemsetAsync(c->done_id[r], 0, (size_t)c->cap * kDoneReplicas * 8, c->stream);
        if (e == hipSuccess)
          e = hipMemsetAsync(c->tiles_done[r], 0, (size_t)kSubCounters * c->cap * 4, c->stream);
        if (e == hipSuccess) e = hipMemsetAsync(c->subs_done[r], 0, (size_t)c->cap * 4, c->stream);
        if (e == hipSuccess && c->trace[r])
          e = hipMemsetAsync(c->trace[r], 0, (size_t)c->cap * sizeof(TraceRec), c->stream);
        if (e == hipSuccess && c->tile_exec[r])
          e = hipMemsetAsync(c->tile_exec[r], 0, (size_t)cfg.tile_counts * 4, c->stream);
      }
    }
    if (!rc && e == hipSuccess) {
      KArgs& a = c->kargs;
      for (int r = 0; r < kRings; ++r) {
        a.hdesc[r] = (const DevDesc*)dev_ptr(c->hdesc[r]);
        a.hends[r] = (const uint64_t*)dev_ptr(c->hends[r]);
        a.ddesc[r] = c->ddesc[r];
        a.dends[r] = c->dends[r];
        a.done_id[r] = c->done_id[r];
        a.tiles_done[r] = c->tiles_done[r];
        a.subs_done[r] = c->subs_done[r];
        a.trace[r] = c->trace[r];
      }
      a.debug = (cfg.tile_counts ? kDebugCount : 0u) | (cfg.jitter << 16);
      a.hctl = (HostCtl*)dev_ptr(c->hctl);
      a.dctl = c->dctl;
      a.cap_mask = c->cap - 1;
      a.ends_mask = 2 * c->cap - 1;
      a.workers = c->workers;
      a.lc_waves = c->lc_waves;
      // s_memrealtime counts at 100 MHz
      a.idle_exit_ticks = cfg.idle_exit_ms == 0xFFFFFFFFu ? 0 : (uint64_t)cfg.idle_exit_ms * 100000u;
      e = hipEventCreate(&c->ev_start);
      if (e == hipSuccess) e = hipEventCreate(&c->ev_end);
      if (e == hipSuccess) rc = launch_kernel(c, 0);
      if (!rc && e == hipSuccess) rc = wait_resident(c);
    }
    if (!rc && e != hipSuccess) rc = fail(GPUOS_EDEVICE, "create: %s", hipGetErrorString(e));
    if (rc) {
      if (c->leaked) return rc;  // the kernel still runs on this memory
      if (c->stream) (void)hipStreamSynchronize(c->stream);
      free_all(c);
      delete c;
      return rc;
    }
  }
  *out = c;
  return 0;
}

}  // namespace

namespace {

int submit_impl(gpuos_ctx* c, const gpuos_op* ops, const gpuos_view* views, uint32_t n, uint64_t* ids_out) {
  if (!c) return fail(GPUOS_EINVAL, "null context");
  if (c->stopped) return fail(GPUOS_ESTATE, "context is stopped");
  if (check_device_error(c)) return fail(GPUOS_ESTATE, "context is poisoned: %s", g_last_error.c_str());
  if (n && !ops) return fail(GPUOS_EINVAL, "ops is null");
  const uint64_t first = c->next_id;
  // validate everything before staging anything
  std::vector<ViewDesc> vd(views ? n : 0);
  for (uint32_t i = 0; i < n; ++i) {
    int rc = validate(ops[i], i, views && views[i].ndim);
    if (rc) return rc;
    if (ops[i].opcode == GPUOS_OP_PROGRAM) {
      const uint32_t pid = (uint32_t)ops[i].aux[0];
      if (pid >= c->programs.size()) return fail(GPUOS_EINVAL, "op %u: unknown program %u", i, pid);
      const uint32_t nin = c->programs[pid].n_inputs();
      for (uint32_t j = 0; j < 3; ++j)
        if ((j < nin) != (ops[i].in[j] != nullptr))
          return fail(GPUOS_EINVAL, "op %u: program %u reads %u inputs: in[%u] must be %s", i, pid, nin, j,
                      j < nin ? "given" : "null");
    }
    if (views && (rc = normalize_view(ops[i], views[i], i, vd[i]))) return rc;
    for (int k = 0; k < 4; ++k) {
      const int64_t dv = ops[i].deps[k];
      if (dv > 0 && (uint64_t)dv >= first + i)
        return fail(GPUOS_EINVAL, "op %u: dependency on id %lld, not yet submitted", i, (long long)dv);
      if (dv < 0 && (uint64_t)(-dv) > i)
        return fail(GPUOS_EINVAL, "op %u: relative dependency %lld points before this call", i,
                    (long long)dv);
    }
    // explicit dependencies must stay in the op's ring
    const uint32_t ring = (ops[i].flags & GPUOS_FLAG_LC) ? 1 : 0;
    if (ring == 1 && c->cfg.priority != 1)
      return fail(GPUOS_EINVAL, "op %u: latency-critical op on a context without the priority ring", i);
    for (int k = 0; k < 4; ++k) {
      const int64_t dv = ops[i].deps[k];
      if (dv < 0) {
        const uint32_t r2 = (ops[i + dv].flags & GPUOS_FLAG_LC) ? 1 : 0;
        if (r2 != ring) return fail(GPUOS_EINVAL, "op %u: explicit dependency across priority rings", i);
      } else if (dv > 0 && !id_retired(c, (uint64_t)dv)) {
        bool known = false;
        const uint32_t r2 = ring_of_id(c, (uint64_t)dv, &known);
        if (known && r2 != ring)
          return fail(GPUOS_EINVAL, "op %u: explicit dependency across priority rings", i);
      }
    }
  }
  auto retired = [c](uint64_t id) { return id_retired(c, id); };
  // geometric growth: reserving exactly size + n on every call would copy the
  // whole staged list on each one-op submit
  if (c->staged.size() + n > c->staged.capacity())
    c->staged.reserve(std::max(2 * c->staged.capacity(), c->staged.size() + n));
  for (uint32_t i = 0; i < n; ++i) {
    Staged& s = c->staged.emplace_back();
    s.op = ops[i];
    if (views) s.view = vd[i];
    s.id = c->next_id++;
    s.ring = (ops[i].flags & GPUOS_FLAG_LC) ? 1 : 0;
    if (ops[i].opcode == GPUOS_OP_PROGRAM) s.prog = c->programs[(uint32_t)ops[i].aux[0]];
    for (int k = 0; k < 4; ++k) {
      const int64_t dv = ops[i].deps[k];
      if (dv > 0) {
        if (!id_retired(c, (uint64_t)dv)) s.deps.push_back((uint64_t)dv);
        ++c->st.deps_explicit;
      } else if (dv < 0) {
        s.deps.push_back(s.id - (uint64_t)(-dv));
        ++c->st.deps_explicit;
      }
    }
    if (c->cfg.auto_deps == 1) {
      const size_t before = s.deps.size();
      const OpRanges R = op_ranges(ops[i], &s.view);
      for (int q = 0; q < R.nr; ++q) {
        const size_t k0 = s.deps.size();
        c->hazards.access(R.r[q], s.id, false, s.deps, retired);
        // GEMV weights (second read range) with no queued writer may be
        // streamed before the op's dependencies complete
        if (ops[i].opcode == GPUOS_OP_GEMV && q == 1 && s.deps.size() == k0)
          s.op.flags |= DF_AUX_READY;
      }
      c->hazards.access(R.w, s.id, true, s.deps, retired);
      // reads recorded above also list this op as a reader of its own output
      // range when it runs in place; drop self-dependencies
      const uint64_t self = s.id;
      s.deps.remove_if([self](uint64_t x) { return x == self; });
      c->st.deps_auto += s.deps.size() - before;
    }
    s.deps.sort_unique();
    c->idseq.push_back(0);
    if (ids_out) ids_out[i] = s.id;
  }
  c->st.ops_submitted += n;
  if ((c->since_prune += n) >= 4096) {
    c->since_prune = 0;
    prune_ids(c);
    c->hazards.prune(retired);
  }
  return 0;
}

}  // namespace

extern "C" {

int gpuos_submit(gpuos_ctx* c, const gpuos_op* ops, uint32_t n, uint64_t* ids_out) {
  return submit_impl(c, ops, nullptr, n, ids_out);
}

int gpuos_submit_views(gpuos_ctx* c, const gpuos_op* ops, const gpuos_view* views, uint32_t n,
                       uint64_t* ids_out) {
  return submit_impl(c, ops, views, n, ids_out);
}

int gpuos_flush(gpuos_ctx* c) {
  if (!c) return fail(GPUOS_EINVAL, "null context");
  if (c->stopped) return fail(GPUOS_ESTATE, "context is stopped");
  return flush_impl(c);
}

int gpuos_submit_flush(gpuos_ctx* c, const gpuos_op* ops, uint32_t n, uint64_t* ids_out) {
  const int rc = submit_impl(c, ops, nullptr, n, ids_out);
  if (rc) return rc;
  return gpuos_flush(c);
}

int gpuos_sync(gpuos_ctx* c, uint64_t upto, int64_t timeout_ns) {
  if (!c) return fail(GPUOS_EINVAL, "null context");
  if (c->exited) return check_device_error(c) ? GPUOS_EDEVICE : 0;
  int rc = flush_impl(c);
  if (rc) return rc;
  if (!c->staged.empty()) return fail(GPUOS_EAGAIN, "sync: ops still staged");
  return sync_impl(c, upto, timeout_ns);
}

int gpuos_query(gpuos_ctx* c, uint64_t id) {
  if (!c) return fail(GPUOS_EINVAL, "null context");
  if (id == 0 || id >= c->next_id) return fail(GPUOS_EINVAL, "query: unknown id");
  if (check_device_error(c)) return GPUOS_EDEVICE;
  if (id_retired(c, id)) return 1;
  const int rc = keep_running(c, false);
  return rc ? rc : 0;
}

int gpuos_get_stats(gpuos_ctx* c, gpuos_stats* out) {
  if (!c || !out) return fail(GPUOS_EINVAL, "null argument");
  c->st.descs_completed = completed_of(c, 0) + completed_of(c, 1);
  c->st.device_error = c->hctl->error;
  c->st.error_desc = c->hctl->error_seq;
  *out = c->st;
  return 0;
}

int gpuos_trace_read(gpuos_ctx* c, gpuos_trace_rec* out, uint32_t max, uint32_t* n_out) {
  if (!c || !n_out) return fail(GPUOS_EINVAL, "null argument");
  *n_out = 0;
  if (c->cfg.trace != 1 || c->host_only) return fail(GPUOS_ESTATE, "tracing is off");
  std::vector<TraceRec> tr((size_t)c->cap * kRings);
  hipStream_t s = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
  for (int r = 0; r < kRings && e == hipSuccess; ++r)
    e = hipMemcpyAsync(tr.data() + (size_t)r * c->cap, c->trace[r], (size_t)c->cap * sizeof(TraceRec),
                       hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (s) (void)hipStreamDestroy(s);
  if (e != hipSuccess) return fail(GPUOS_EDEVICE, "trace copy: %s", hipGetErrorString(e));
  std::vector<gpuos_trace_rec> recs;
  for (int r = 0; r < kRings; ++r) {
    const uint64_t done = completed_of(c, r);
    const uint64_t lo = done > c->cap ? done - c->cap + 1 : 1;
    for (uint64_t sq = lo; sq <= done; ++sq) {
      const TraceRec& t = tr[(size_t)r * c->cap + ((sq - 1) & (c->cap - 1))];
      if (t.seq != sq) continue;
      gpuos_trace_rec o;
      o.seq = sq;
      o.t_claim = t.t_claim;
      o.t_done = t.t_done;
      o.t_wait = t.t_wait;
      o.t_end = t.t_end;
      o.t_ack = t.t_ack;
      o.opcode = t.opcode;
      o.ntiles = t.ntiles;
      o.ring = (uint32_t)r;
      o.first_ops = c->hdesc[r][(sq - 1) & (c->cap - 1)].seq == sq
                        ? c->hdesc[r][(sq - 1) & (c->cap - 1)].user_ops
                        : 0;
      recs.push_back(o);
    }
  }
  const size_t k = std::min<size_t>(recs.size(), max);
  if (out) memcpy(out, recs.data() + (recs.size() - k), k * sizeof(gpuos_trace_rec));
  *n_out = (uint32_t)k;
  return 0;
}

int gpuos_stop(gpuos_ctx* c, int64_t timeout_ns) {
  if (!c) return fail(GPUOS_EINVAL, "null context");
  if (c->host_only) {  // nothing runs; the context still stops accepting work
    c->stopped = true;
    return 0;
  }
  if (c->exited) return 0;
  if (c->parked && c->staged.empty()) {  // not running and nothing to run
    c->stopped = true;
    c->exited = true;
    return check_device_error(c) ? GPUOS_EDEVICE : 0;
  }
  if (c->leaked) return fail(GPUOS_ETIMEDOUT, "resident kernel did not exit");
  int rc = 0;
  if (!c->stopped) {
    if (!c->poisoned) {
      int r2 = flush_impl(c);
      if (!r2) r2 = sync_impl(c, 0, timeout_ns);
      if (r2) rc = r2;
    }
    c->staged.clear();
    c->stopped = true;
    // every published descriptor retires before the kernel lets its waves go
    std::atomic_thread_fence(std::memory_order_release);
    store_rel(&c->hctl->stop_req, 1);
  }
  // wait for the kernel to exit (it may already have left after idling)
  const int r3 = wait_kernel_end(c, timeout_ns);
  if (r3) return r3;
  c->exited = true;
  account_launch(c);
  if (check_device_error(c)) return GPUOS_EDEVICE;
  return rc;
}

int gpuos_program_define(gpuos_ctx* c, const gpuos_program* prog, uint32_t* id_out) {
  if (!c || !id_out) return fail(GPUOS_EINVAL, "null argument");
  if (c->stopped) return fail(GPUOS_ESTATE, "context is stopped");
  if (c->programs.size() >= GPUOS_PROG_MAX_PROGRAMS)
    return fail(GPUOS_EINVAL, "more than %d programs", GPUOS_PROG_MAX_PROGRAMS);
  ProgCode pc;
  const int rc = check_program(prog, pc);
  if (rc) return rc;
  *id_out = (uint32_t)c->programs.size();
  c->programs.push_back(pc);
  return 0;
}

int gpuos_program_update(gpuos_ctx* c, uint32_t id, const gpuos_program* prog) {
  if (!c) return fail(GPUOS_EINVAL, "null context");
  if (c->stopped) return fail(GPUOS_ESTATE, "context is stopped");
  if (id >= c->programs.size()) return fail(GPUOS_EINVAL, "unknown program %u", id);
  ProgCode pc;
  const int rc = check_program(prog, pc);
  if (rc) return rc;
  // staged and published ops keep the body they were submitted with
  c->programs[id] = pc;
  return 0;
}

int gpuos_program_compile(gpuos_ctx* c, const uint32_t* ids, uint32_t n_ids, uint32_t dtypes,
                          char* log, size_t log_bytes) {
  if (log && log_bytes) log[0] = '\0';
  if (!c) return fail(GPUOS_EINVAL, "null context");
  if (c->stopped) return fail(GPUOS_ESTATE, "context is stopped");
  if (c->static_mem) return fail(GPUOS_ESTATE, "a static context allocates nothing: it cannot load compiled code");
  const uint32_t all = (1u << GPUOS_F32) | (1u << GPUOS_BF16) | (1u << GPUOS_F16);
  if (dtypes == 0) dtypes = all;
  if (dtypes & ~all) return fail(GPUOS_EINVAL, "dtypes mask 0x%x has bits other than F32, BF16, F16", dtypes);
  std::vector<uint32_t> list;
  if (ids) {
    for (uint32_t i = 0; i < n_ids; ++i) {
      if (ids[i] >= c->programs.size()) return fail(GPUOS_EINVAL, "unknown program %u", ids[i]);
      list.push_back(ids[i]);
    }
  } else {
    for (uint32_t i = 0; i < (uint32_t)c->programs.size(); ++i) list.push_back(i);
  }
  if (list.empty()) return fail(GPUOS_EINVAL, "no program to compile");
  auto m = std::make_shared<RtcModule>();
  m->dtypes = dtypes;
  std::string bodies = "// Program bodies of one gpuos_program_compile call (generated).\n#pragma once\n";
  char buf[96];
  snprintf(buf, sizeof buf, "#define GPUOS_RTC_DTYPES 0x%xu\n", dtypes);
  bodies += buf;
  bodies += "namespace gpuos {\n";
  std::string cases;
  for (uint32_t id : list) {
    const ProgCode& pc = c->programs[id];
    const std::string key = body_key(pc);
    if (m->index.count(key)) continue;
    const uint32_t k = (uint32_t)m->index.size();
    if (k == GPUOS_PROG_MAX_COMPILED)
      return fail(GPUOS_EINVAL, "more than %d distinct bodies in one compile", GPUOS_PROG_MAX_COMPILED);
    m->index.emplace(key, k);
    emit_body(bodies, k, pc);
    cases += " X(" + std::to_string(k) + ")";
  }
  bodies += "}  // namespace gpuos\n#define GPUOS_RTC_BODIES(X)" + cases + "\n";
  c->rtc_source = bodies;
  std::vector<char> code;
  std::string clog;
  int rc = rtc_compile(c->host_only ? std::string("gfx950") : c->arch, bodies, code, clog);
  if (log && log_bytes) {
    const size_t k = std::min(clog.size(), log_bytes - 1);
    memcpy(log, clog.data(), k);
    log[k] = '\0';
  }
  if (rc) return rc;
  if (!c->host_only) {
    rc = rtc_load(c, code, *m);
    if (rc) return rc;
  }
  c->rtc_new = std::move(m);  // the previous compile stays loaded while a kernel runs it
  return 0;
}

int gpuos_yield(gpuos_ctx* c, int64_t timeout_ns) {
  if (!c) return fail(GPUOS_EINVAL, "null context");
  if (c->stopped) return fail(GPUOS_ESTATE, "context is stopped");
  if (c->host_only || c->exited || c->parked) return 0;
  int rc = flush_impl(c);
  if (!rc) rc = sync_impl(c, 0, timeout_ns);
  if (rc) return rc;
  return park_kernel(c, timeout_ns);
}

int gpuos_destroy(gpuos_ctx* c, int64_t timeout_ns) {
  if (!c) return fail(GPUOS_EINVAL, "null context");
  int rc = 0;
  if (!c->host_only) {
    rc = gpuos_stop(c, timeout_ns);
    if (c->leaked) {
      // never free memory (or unload code) a running kernel may still touch
      if (c->rtc_run) c->rtc_run->leak = true;
      rc = fail(GPUOS_ETIMEDOUT, "resident kernel did not exit; its memory is leaked");
      delete c;
      return rc;
    }
  }
  free_all(c);
  delete c;
  return rc;
}

// ---------------------------------------------------------------------------
// per-op launch comparator

}  // extern "C"

namespace {

// Checks ops[0, n) and returns the compute-unit count of `device`.  Makes no
// stream call, so it may run before a capture begins.
int per_op_prepare(int device, const gpuos_op* ops, uint32_t n, uint32_t* cus) {
  if (n && !ops) return fail(GPUOS_EINVAL, "ops is null");
  for (uint32_t i = 0; i < n; ++i) {
    int rc = validate(ops[i], i);
    if (rc) return rc;
    if (ops[i].opcode == GPUOS_OP_PROGRAM)
      return fail(GPUOS_EINVAL, "op %u: PROGRAM ops run only in a context (their bodies belong to it)", i);
  }
  static thread_local int cached_dev = -2;
  static thread_local uint32_t cached_cus = 0;
  if (cached_dev != device) {
    hipDeviceProp_t prop;
    HIP_TRY(hipGetDeviceProperties(&prop, device));
    cached_cus = (uint32_t)prop.multiProcessorCount;
    cached_dev = device;
  }
  *cus = cached_cus;
  HIP_TRY(hipSetDevice(device));
  return 0;
}

// Issues the per-op launches of ops[0, n) (already checked by per_op_prepare)
// on stream s: one gpuos_single launch per op, or per fused group if fuse.
int issue_per_op(const gpuos_op* ops, uint32_t n, int fuse, uint32_t cus, hipStream_t s) {
  gpuos_ctx tmp;  // host-side planning state only
  tmp.host_only = true;
  gpuos_config_default(&tmp.cfg);
  tmp.cfg.fusion = fuse ? 1 : 2;
  tmp.workers = cus * 16;
  tmp.spread_big = true;
  if (!fuse) {
    DevDesc d;
    for (uint32_t i = 0; i < n; ++i) {
      encode_plain(ops[i], tmp.cfg, tmp.workers, d, true);
      mark_streaming(tmp.cfg, d);
      if (ops[i].opcode == GPUOS_OP_NOP) continue;
      HIP_TRY(launch_single(d, nullptr, s));
    }
    return 0;
  }
  tmp.staged.reserve(n);
  for (uint32_t i = 0; i < n; ++i) {
    Staged& st = tmp.staged.emplace_back();
    st.op = ops[i];
    st.id = i + 1;
    st.ring = 0;
  }
  std::vector<Planned> plan;
  plan.reserve(n);
  plan_ops(&tmp, 0, tmp.staged.size(), plan);
  for (Planned& pl : plan) {
    if (pl.desc.opcode == GPUOS_OP_NOP) continue;
    HIP_TRY(launch_single(pl.desc, nullptr, s));
  }
  return 0;
}

}  // namespace

struct gpuos_graph {
  int device = 0;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

extern "C" {

int gpuos_baseline_run(int device, const gpuos_op* ops, uint32_t n, int fuse, void* stream) {
  uint32_t cus = 0;
  int rc = per_op_prepare(device, ops, n, &cus);
  if (rc) return rc;
  return issue_per_op(ops, n, fuse, cus, reinterpret_cast<hipStream_t>(stream));
}

int gpuos_graph_create(int device, const gpuos_op* ops, uint32_t n, int fuse, gpuos_graph** out) {
  if (!out) return fail(GPUOS_EINVAL, "out is null");
  *out = nullptr;
  uint32_t cus = 0;
  int rc = per_op_prepare(device, ops, n, &cus);
  if (rc) return rc;
  hipStream_t s = nullptr;
  HIP_TRY(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
  auto* g = new gpuos_graph();
  g->device = device;
  hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    rc = issue_per_op(ops, n, fuse, cus, s);
    const hipError_t e2 = hipStreamEndCapture(s, &g->graph);
    if (!rc && e2 != hipSuccess) e = e2;
  }
  if (!rc && e == hipSuccess) e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
  (void)hipStreamDestroy(s);
  if (rc || e != hipSuccess) {
    if (!rc) rc = fail(GPUOS_EDEVICE, "graph capture: %s", hipGetErrorString(e));
    if (g->exec) (void)hipGraphExecDestroy(g->exec);
    if (g->graph) (void)hipGraphDestroy(g->graph);
    delete g;
    return rc;
  }
  *out = g;
  return 0;
}

int gpuos_graph_launch(gpuos_graph* g, void* stream) {
  if (!g) return fail(GPUOS_EINVAL, "null graph");
  HIP_TRY(hipSetDevice(g->device));
  HIP_TRY(hipGraphLaunch(g->exec, reinterpret_cast<hipStream_t>(stream)));
  return 0;
}

int gpuos_graph_destroy(gpuos_graph* g) {
  if (!g) return fail(GPUOS_EINVAL, "null graph");
  int rc = 0;
  if (g->exec && hipGraphExecDestroy(g->exec) != hipSuccess) rc = fail(GPUOS_EDEVICE, "graph exec destroy");
  if (g->graph && hipGraphDestroy(g->graph) != hipSuccess) rc = fail(GPUOS_EDEVICE, "graph destroy");
  delete g;
  return rc;
}

int gpuos_launch_overhead(int device, uint32_t n, double* async_us, double* sync_us) {
  if (n == 0 || !async_us || !sync_us) return fail(GPUOS_EINVAL, "launch_overhead: n = 0 or a null output");
  HIP_TRY(hipSetDevice(device));
  hipStream_t s = nullptr;
  HIP_TRY(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
  int rc = 0;
  auto run = [&]() -> int {
    for (int i = 0; i < 100; ++i)
      if (launch_empty(s) != hipSuccess) return fail(GPUOS_EDEVICE, "empty kernel launch failed");
    if (hipStreamSynchronize(s) != hipSuccess) return fail(GPUOS_EDEVICE, "stream synchronize failed");
    auto t0 = std::chrono::steady_clock::now();
    for (uint32_t i = 0; i < n; ++i)
      if (launch_empty(s) != hipSuccess) return fail(GPUOS_EDEVICE, "empty kernel launch failed");
    if (hipStreamSynchronize(s) != hipSuccess) return fail(GPUOS_EDEVICE, "stream synchronize failed");
    auto t1 = std::chrono::steady_clock::now();
    *async_us = std::chrono::duration<double, std::micro>(t1 - t0).count() / n;
    t0 = std::chrono::steady_clock::now();
    for (uint32_t i = 0; i < n; ++i) {
      if (launch_empty(s) != hipSuccess) return fail(GPUOS_EDEVICE, "empty kernel launch failed");
      if (hipStreamSynchronize(s) != hipSuccess) return fail(GPUOS_EDEVICE, "stream synchronize failed");
    }
    t1 = std::chrono::steady_clock::now();
    *sync_us = std::chrono::duration<double, std::micro>(t1 - t0).count() / n;
    return 0;
  };
  rc = run();
  (void)hipStreamDestroy(s);
  return rc;
}

// ---------------------------------------------------------------------------
// debug hooks

int gpuos_debug_read_desc(gpuos_ctx* c, int ring, uint64_t seq, void* out) {
  if (!c || !out || ring < 0 || ring >= kRings) return fail(GPUOS_EINVAL, "bad argument");
  if (seq == 0 || seq > c->pub_seq[ring] || (c->pub_seq[ring] >= c->cap && seq <= c->pub_seq[ring] - c->cap))
    return fail(GPUOS_EINVAL, "sequence %llu not in the ring", (unsigned long long)seq);
  memcpy(out, &c->hdesc[ring][(seq - 1) & (c->cap - 1)], sizeof(DevDesc));
  return 0;
}

uint64_t gpuos_debug_published(gpuos_ctx* c, int ring) {
  if (!c || ring < 0 || ring >= kRings) return 0;
  return c->pub_seq[ring];
}

int gpuos_debug_seq_of(gpuos_ctx* c, uint64_t id, int* ring_out, uint64_t* seq_out) {
  if (!c || !ring_out || !seq_out) return fail(GPUOS_EINVAL, "bad argument");
  if (id == 0 || id >= c->next_id || id < c->id_base) return fail(GPUOS_EINVAL, "unknown id");
  const uint64_t v = c->idseq[id - c->id_base];
  if (!v) return fail(GPUOS_EAGAIN, "id still staged");
  *ring_out = (int)(v >> 63);
  *seq_out = v & ((1ull << 63) - 1);
  return 0;
}

size_t gpuos_debug_rtc_source(gpuos_ctx* c, char* buf, size_t n) {
  if (!c) return 0;
  if (buf && n) {
    const size_t k = std::min(c->rtc_source.size(), n - 1);
    memcpy(buf, c->rtc_source.data(), k);
    buf[k] = '\0';
  }
  return c->rtc_source.size() + 1;
}

int gpuos_debug_tile_counts(gpuos_ctx* c, int ring, uint32_t* out, uint32_t n) {
  if (!c || !out || ring < 0 || ring >= kRings) return fail(GPUOS_EINVAL, "bad argument");
  if (c->host_only || !c->tile_exec[ring]) return fail(GPUOS_ESTATE, "tile counting is off");
  if (n > c->cfg.tile_counts) return fail(GPUOS_EINVAL, "n above config.tile_counts");
  hipStream_t s = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipMemcpyAsync(out, c->tile_exec[ring], (size_t)n * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (s) (void)hipStreamDestroy(s);
  if (e != hipSuccess) return fail(GPUOS_EDEVICE, "tile count copy: %s", hipGetErrorString(e));
  return 0;
}

int gpuos_debug_consumer_attach(gpuos_ctx* c) {
  if (!c) return fail(GPUOS_EINVAL, "bad argument");
  if (!c->host_only) return fail(GPUOS_ESTATE, "only host-only contexts take a host consumer");
  c->consumer = true;
  return 0;
}

// The consumer side touches only what the device would: the published tails,
// the ring slots and the retire cursors, never the producer's own fields.
uint64_t gpuos_debug_consumer_tail(gpuos_ctx* c, int ring) {
  if (!c || !c->host_only || ring < 0 || ring >= kRings) return 0;
  return load_acq(&c->hctl->tail[ring]);
}

int gpuos_debug_consumer_read(gpuos_ctx* c, int ring, uint64_t seq, void* out) {
  if (!c || !out || ring < 0 || ring >= kRings || seq == 0) return fail(GPUOS_EINVAL, "bad argument");
  if (!c->host_only) return fail(GPUOS_ESTATE, "only host-only contexts take a host consumer");
  const DevDesc* d = &c->hdesc[ring][(seq - 1) & (c->cap - 1)];
  if (d->seq != seq || d->check != ((uint32_t)seq ^ kDescMagic))
    return fail(GPUOS_EINVAL, "slot of sequence %llu holds sequence %llu",
                (unsigned long long)seq, (unsigned long long)d->seq);
  memcpy(out, d, sizeof(DevDesc));
  return 0;
}

int gpuos_debug_consumer_retire(gpuos_ctx* c, int ring, uint64_t upto) {
  if (!c || ring < 0 || ring >= kRings) return fail(GPUOS_EINVAL, "bad argument");
  if (!c->host_only) return fail(GPUOS_ESTATE, "only host-only contexts take a host consumer");
  if (upto > load_acq(&c->hctl->tail[ring]))
    return fail(GPUOS_EINVAL, "retire beyond the published tail");
  if (upto > load_acq(&c->hctl->completed[ring])) store_rel(&c->hctl->completed[ring], upto);
  return 0;
}

int gpuos_debug_retire(gpuos_ctx* c, int ring, uint64_t upto) {
  if (!c || ring < 0 || ring >= kRings) return fail(GPUOS_EINVAL, "bad argument");
  if (!c->host_only) return fail(GPUOS_ESTATE, "only host-only contexts are retired by hand");
  if (upto > c->pub_seq[ring]) return fail(GPUOS_EINVAL, "beyond the last published sequence");
  if (upto > c->hctl->completed[ring]) store_rel(&c->hctl->completed[ring], upto);
  return 0;
}

}  // extern "C"
