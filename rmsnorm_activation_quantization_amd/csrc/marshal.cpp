// Argument marshalling of the library's entry points for the Python binding
// (the CPython module _marshal): the fused row calls, the unfused sequence's
// launches and the QK calls.
//
// The binding's checks, the allocation of missing outputs and the call of the
// C entry point (with the tensors' device current, as torch's own operators
// do), done on torch's C++ tensors.  From Python every tensor
// attribute a check reads is a call into torch of 0.1-0.4 us, and an eager
// decode-sized call is bound by that host time; here the same reads cost
// nanoseconds.  Nothing here computes: every step of the method runs in the
// library's kernels, reached through the C ABI (include/rmsnorm_quant.h) by
// function pointers that the Python binding resolves from the library it has
// loaded (so that a test can point the binding at another build of it).
//
// rows(), quantize() and qk() return the outputs as a tuple when the C call returns RQ_OK
// and the status code (an int) otherwise; arguments the checks refuse raise
// ValueError, with the Python binding's messages.

#include <Python.h>

#include <ATen/core/Tensor.h>
#include <ATen/ops/empty.h>
#include <c10/core/DeviceGuard.h>
#include <c10/hip/HIPStream.h>
#include <torch/csrc/autograd/python_variable.h>

#include <algorithm>
#include <cstdint>
#include <initializer_list>
#include <string>
#include <utility>
#include <vector>

namespace {

// What rows() runs (the binding passes one of these with the entry points);
// quantize() takes the first three.
enum RowOp { kFp8Token = 0, kFp8Group = 1, kMxfp4 = 2, kFp8GroupT = 3, kMxfp4T = 4, kNorm = 5 };
// What qk() runs.
enum QkOp { kQkBf16 = 0, kQkFp8 = 1, kQkMxfp4 = 2 };

using RowFn = int (*)(const void*, int64_t, const void*, int64_t, const void*, int64_t, int64_t, float, void*, void*,
                      void*, void*, void*);
using RowGroupFn = int (*)(const void*, int64_t, const void*, int64_t, const void*, int64_t, int64_t, float, int64_t,
                           void*, void*, void*, void*, void*);
using RowTFn = int (*)(const void*, int64_t, const void*, int64_t, const void*, int64_t, int64_t, float, void*, void*,
                       void*, int64_t, void*, void*);
using RowGroupTFn = int (*)(const void*, int64_t, const void*, int64_t, const void*, int64_t, int64_t, float, int64_t,
                            void*, void*, void*, int64_t, void*, void*);
using QuantFn = int (*)(const void*, int64_t, int64_t, int64_t, void*, void*, void*);
using QuantGroupFn = int (*)(const void*, int64_t, int64_t, int64_t, int64_t, void*, void*, void*);
using NormFn = int (*)(const void*, int64_t, const void*, int64_t, const void*, int64_t, int64_t, float, void*, void*,
                       void*);
using QkFn = int (*)(const void*, int64_t, const void*, int64_t, const void*, const void*, int64_t, int64_t, int64_t,
                     int64_t, float, void*, void*, void*, void*);
using QkQuantFn = int (*)(const void*, int64_t, const void*, int64_t, const void*, const void*, int64_t, int64_t,
                          int64_t, int64_t, float, void*, void*, void*, void*, void*, void*);

struct Refused {  // raised as ValueError
  std::string msg;
};

std::string dtype_name(c10::ScalarType t) {
  switch (t) {
    case at::kBFloat16: return "torch.bfloat16";
    case at::kHalf: return "torch.float16";
    case at::kFloat: return "torch.float32";
    case at::kByte: return "torch.uint8";
    case at::kFloat8_e4m3fn: return "torch.float8_e4m3fn";
    default: return c10::toString(t);
  }
}

std::string shape_str(at::IntArrayRef s) {
  std::string r = "[";
  for (size_t i = 0; i < s.size(); ++i) r += (i ? ", " : "") + std::to_string(s[i]);
  return r + "]";
}

// Python's floor division, for sizes the caller may have given negative.
int64_t floordiv(int64_t a, int64_t b) {
  const int64_t q = a / b;
  return (a % b != 0 && ((a < 0) != (b < 0))) ? q - 1 : q;
}

// A tensor argument (borrowed from the caller's object for the call), or null
// for None where None is allowed.
const at::Tensor* tensor_arg(PyObject* o, const char* name, bool optional) {
  if (o == Py_None && optional) return nullptr;
  if (!THPVariable_Check(o)) throw Refused{std::string(name) + " must be a tensor"};
  return &THPVariable_Unpack(o);
}

// Row stride (elements) of a 2-D bf16 or fp16 CUDA tensor with unit column
// stride, of dtype `dt` when one is given.
int64_t row_stride(const at::Tensor& t, const char* name, const c10::ScalarType* dt) {
  const c10::ScalarType st = t.scalar_type();
  if (t.dim() != 2 || (st != at::kBFloat16 && st != at::kHalf) || !t.is_cuda())
    throw Refused{std::string(name) + " must be a 2-D bfloat16 or float16 CUDA tensor"};
  if (dt != nullptr && st != *dt) throw Refused{std::string(name) + " must have the dtype of x (" + dtype_name(*dt) + ")"};
  if (t.size(1) > 1 && t.stride(1) != 1) throw Refused{std::string(name) + " must have unit column stride"};
  return t.size(0) > 1 ? t.stride(0) : t.size(1);
}

// The kernels dereference every pointer on the device of the first input, so
// a host tensor or one on another GPU is refused.
void same_device(const at::Tensor* t, const char* name, const c10::Device& dev) {
  if (t != nullptr && t->device() != dev)
    throw Refused{std::string(name) + " is on " + t->device().str() + "; every tensor must be on " + dev.str()};
}

// A caller-supplied output: the exact shape, one of the dtypes, contiguous, on
// `dev`.  The library cannot see buffer sizes, so a wrong output tensor is
// refused here rather than written past its end.
const at::Tensor& checked_out(const at::Tensor& t, at::IntArrayRef shape, std::initializer_list<c10::ScalarType> dts,
                              const char* name, const c10::Device& dev) {
  const bool dt_ok = std::find(dts.begin(), dts.end(), t.scalar_type()) != dts.end();
  if (t.sizes() != shape || !dt_ok || !t.is_contiguous() || t.device() != dev)
    throw Refused{std::string(name) + " must be a contiguous " + shape_str(shape) + " " + dtype_name(*dts.begin()) +
                  " tensor on " + dev.str()};
  return t;
}

// The caller's stream (a torch.cuda.Stream, or anything with an integer
// `cuda_stream`, on the tensors' device when it says which), else torch's
// current stream on that device.
void* stream_of(PyObject* stream, const c10::Device& dev) {
  if (stream == Py_None) return c10::hip::getCurrentHIPStream(dev.index()).stream();
  PyObject* s = PyObject_GetAttrString(stream, "cuda_stream");
  void* p = s != nullptr ? PyLong_AsVoidPtr(s) : nullptr;
  Py_XDECREF(s);
  if (PyErr_Occurred()) {
    PyErr_Clear();
    throw Refused{"stream must be a torch.cuda.Stream"};
  }
  if (PyObject* d = PyObject_GetAttrString(stream, "device_index")) {
    const long idx = PyLong_Check(d) ? PyLong_AsLong(d) : (long)dev.index();
    Py_DECREF(d);
    if (idx != (long)dev.index())
      throw Refused{"stream is on cuda:" + std::to_string(idx) + "; every tensor is on " + dev.str()};
  }
  PyErr_Clear();  // no device_index: nothing to compare
  return p;
}

PyObject* wrap(const at::Tensor& t) { return THPVariable_Wrap(t); }

// The codes and scales outputs of a row format (kFp8Token ... kMxfp4T): the
// caller's, checked, or new ones.  Column-major scales are [rows, n >= M]
// with unit column stride (a view of a wider buffer is fine); their row
// stride is ld_scale.
struct Codes {
  at::Tensor q, sc;
  int64_t ld_scale = 0;
};
Codes codes_and_scales(int op, const at::Tensor* qo, const at::Tensor* so, int64_t M, int64_t H, int64_t group,
                       const at::TensorOptions& opt, const c10::Device& dev) {
  Codes c;
  const int64_t G = group > 0 ? std::max<int64_t>(floordiv(H, group), 1) : 1;
  const int64_t B = std::max<int64_t>(floordiv(H, 32), 1);
  if (op == kFp8Token || op == kFp8Group || op == kFp8GroupT)
    c.q = qo != nullptr ? checked_out(*qo, {M, H}, {at::kByte, at::kFloat8_e4m3fn}, "q_out", dev)
                        : at::empty({M, H}, opt.dtype(at::kFloat8_e4m3fn));
  else if (op == kMxfp4 || op == kMxfp4T)
    c.q = qo != nullptr ? checked_out(*qo, {M, floordiv(H, 2)}, {at::kByte}, "q_out", dev)
                        : at::empty({M, floordiv(H, 2)}, opt.dtype(at::kByte));
  if (op == kFp8Token) {
    if (so == nullptr) {
      c.sc = at::empty({M, 1}, opt.dtype(at::kFloat));
    } else {
      const bool ok = (so->dim() == 1 && so->size(0) == M) || (so->dim() == 2 && so->size(0) == M && so->size(1) == 1);
      if (!ok)
        throw Refused{"scale_out must be a contiguous [" + std::to_string(M) + "] or [" + std::to_string(M) +
                      ", 1] float32 tensor"};
      c.sc = checked_out(*so, so->sizes(), {at::kFloat}, "scale_out", dev);
    }
  } else if (op == kFp8Group) {
    c.sc = so != nullptr ? checked_out(*so, {M, G}, {at::kFloat}, "scale_out", dev)
                         : at::empty({M, G}, opt.dtype(at::kFloat));
  } else if (op == kMxfp4) {
    c.sc = so != nullptr ? checked_out(*so, {M, B}, {at::kByte}, "scale_out", dev)
                         : at::empty({M, B}, opt.dtype(at::kByte));
  } else if (op == kFp8GroupT || op == kMxfp4T) {
    const int64_t srows = op == kFp8GroupT ? G : B;
    const c10::ScalarType sdt = op == kFp8GroupT ? at::kFloat : at::kByte;
    if (so == nullptr) {
      c.sc = at::empty({srows, std::max<int64_t>(M, 1)}, opt.dtype(sdt));
      c.ld_scale = std::max<int64_t>(M, 1);
    } else {
      if (so->dim() != 2 || so->size(0) != srows || so->size(1) < M || so->scalar_type() != sdt ||
          (so->size(1) > 1 && so->stride(1) != 1) || so->device() != dev)
        throw Refused{"scale_out must be a [" + std::to_string(srows) + ", >= " + std::to_string(M) + "] " +
                      dtype_name(sdt) + " tensor with unit column stride"};
      c.sc = *so;
      c.ld_scale = srows > 1 ? so->stride(0) : std::max<int64_t>(so->size(1), 1);
    }
  }
  return c;
}

// FP8 codes come back as float8_e4m3fn (a caller's uint8 buffer is viewed),
// per-token scales as [M, 1].
PyObject* codes_tuple_items(int op, at::Tensor& q, at::Tensor& sc, int64_t M, PyObject** q_obj) {
  if (q.scalar_type() == at::kByte && op != kMxfp4 && op != kMxfp4T) q = q.view(at::kFloat8_e4m3fn);
  if (op == kFp8Token && sc.dim() == 1) sc = sc.view({M, 1});
  *q_obj = wrap(q);
  return wrap(sc);
}

PyObject* rows_impl(PyObject* const* a) {
  const int op = (int)PyLong_AsLong(a[0]);
  PyObject* fns = a[1];  // (bf16 entry point, fp16 entry point) as addresses
  const at::Tensor& x = *tensor_arg(a[2], "x", false);
  const at::Tensor& res = *tensor_arg(a[3], "residual", false);
  const at::Tensor& w = *tensor_arg(a[4], "weight", false);
  const float eps = (float)PyFloat_AsDouble(a[5]);
  const int64_t group = PyLong_AsLongLong(a[6]);
  const at::Tensor* ro = tensor_arg(a[7], "residual_out", true);
  const at::Tensor* qo = tensor_arg(a[8], "q_out", true);
  const at::Tensor* so = tensor_arg(a[9], "scale_out", true);
  const int emit_y = PyObject_IsTrue(a[10]);
  const at::Tensor* yo = tensor_arg(a[11], "y_out", true);
  if (PyErr_Occurred() || !PyTuple_Check(fns) || PyTuple_GET_SIZE(fns) != 2) {
    if (!PyErr_Occurred()) PyErr_SetString(PyExc_TypeError, "rows: the entry points must be a pair");
    return nullptr;
  }

  // inputs: one element type, one device
  const int64_t ldx = row_stride(x, "x", nullptr);
  const c10::ScalarType dt = x.scalar_type();
  const int64_t ldr = row_stride(res, "residual", &dt);
  const int64_t M = x.size(0), H = x.size(1);
  if (res.sizes() != x.sizes() || w.dim() != 1 || w.size(0) != H || res.scalar_type() != dt || w.scalar_type() != dt)
    throw Refused{"residual must be [M, H] and weight [H], both " + dtype_name(dt) + " like x"};
  if (!w.is_contiguous()) throw Refused{"weight must be contiguous"};
  const c10::Device dev = x.device();
  same_device(&res, "residual", dev);
  same_device(&w, "weight", dev);
  same_device(ro, "residual_out", dev);
  same_device(yo, "y_out", dev);
  for (const auto& [name, t] : {std::pair<const char*, const at::Tensor*>{"residual_out", ro}, {"y_out", yo}}) {
    if (t != nullptr && (t->sizes() != x.sizes() || t->scalar_type() != dt || !t->is_contiguous()))
      throw Refused{std::string(name) + " must be a contiguous [M, H] " + dtype_name(dt) + " tensor"};
  }
  const auto opt = x.options();
  const at::Tensor r_out = ro != nullptr ? *ro : at::empty({M, H}, opt);
  at::Tensor y_out;
  if (yo != nullptr)
    y_out = *yo;
  else if (emit_y || op == kNorm)
    y_out = at::empty({M, H}, opt);

  Codes c = codes_and_scales(op, qo, so, M, H, group, opt, dev);
  at::Tensor& q = c.q;
  at::Tensor& sc = c.sc;
  const int64_t ld_scale = c.ld_scale;

  void* fn = PyLong_AsVoidPtr(PyTuple_GET_ITEM(fns, dt == at::kHalf ? 1 : 0));
  if (PyErr_Occurred()) return nullptr;
  const c10::DeviceGuard on_device(dev);  // the library checks and launches on the current device
  void* stream = stream_of(a[12], dev);
  const void *xp = x.data_ptr(), *rp = res.data_ptr(), *wp = w.data_ptr();
  void* rop = r_out.data_ptr();
  void* yp = y_out.defined() ? y_out.data_ptr() : nullptr;
  int st = 0;
  switch (op) {
    case kFp8Token:
    case kMxfp4:
      st = reinterpret_cast<RowFn>(fn)(xp, ldx, rp, ldr, wp, M, H, eps, rop, q.data_ptr(), sc.data_ptr(), yp, stream);
      break;
    case kFp8Group:
      st = reinterpret_cast<RowGroupFn>(fn)(xp, ldx, rp, ldr, wp, M, H, eps, group, rop, q.data_ptr(), sc.data_ptr(),
                                             yp, stream);
      break;
    case kFp8GroupT:
      st = reinterpret_cast<RowGroupTFn>(fn)(xp, ldx, rp, ldr, wp, M, H, eps, group, rop, q.data_ptr(), sc.data_ptr(),
                                              ld_scale, yp, stream);
      break;
    case kMxfp4T:
      st = reinterpret_cast<RowTFn>(fn)(xp, ldx, rp, ldr, wp, M, H, eps, rop, q.data_ptr(), sc.data_ptr(), ld_scale,
                                         yp, stream);
      break;
    case kNorm:
      st = reinterpret_cast<NormFn>(fn)(xp, ldx, rp, ldr, wp, M, H, eps, rop, yp, stream);
      break;
    default:
      PyErr_SetString(PyExc_ValueError, "rows: unknown operation");
      return nullptr;
  }
  if (st != 0) return PyLong_FromLong(st);
  if (op == kNorm) return Py_BuildValue("(NN)", wrap(r_out), wrap(y_out));
  PyObject* q_obj;
  PyObject* sc_obj = codes_tuple_items(op, q, sc, M, &q_obj);
  PyObject* y_obj = y_out.defined() ? wrap(y_out) : (Py_INCREF(Py_None), Py_None);
  return Py_BuildValue("(NNNN)", q_obj, wrap(r_out), sc_obj, y_obj);
}

// The quantize launch of the unfused sequence: y (a 2-D bf16 or fp16 tensor)
// to codes and scales in one of the three row formats.
PyObject* quantize_impl(PyObject* const* a) {
  const int op = (int)PyLong_AsLong(a[0]);
  PyObject* fns = a[1];
  const at::Tensor& y = *tensor_arg(a[2], "y", false);
  const int64_t group = PyLong_AsLongLong(a[3]);
  const at::Tensor* qo = tensor_arg(a[4], "q_out", true);
  const at::Tensor* so = tensor_arg(a[5], "scale_out", true);
  if (PyErr_Occurred() || !PyTuple_Check(fns) || PyTuple_GET_SIZE(fns) != 2 || op < kFp8Token || op > kMxfp4) {
    if (!PyErr_Occurred()) PyErr_SetString(PyExc_TypeError, "quantize: an operation and a pair of entry points");
    return nullptr;
  }
  const int64_t ldy = row_stride(y, "y", nullptr);
  const int64_t M = y.size(0), H = y.size(1);
  const c10::Device dev = y.device();
  Codes c = codes_and_scales(op, qo, so, M, H, group, y.options(), dev);
  void* fn = PyLong_AsVoidPtr(PyTuple_GET_ITEM(fns, y.scalar_type() == at::kHalf ? 1 : 0));
  if (PyErr_Occurred()) return nullptr;
  const c10::DeviceGuard on_device(dev);
  void* stream = stream_of(a[6], dev);
  const int st = op == kFp8Group
      ? reinterpret_cast<QuantGroupFn>(fn)(y.data_ptr(), ldy, M, H, group, c.q.data_ptr(), c.sc.data_ptr(), stream)
      : reinterpret_cast<QuantFn>(fn)(y.data_ptr(), ldy, M, H, c.q.data_ptr(), c.sc.data_ptr(), stream);
  if (st != 0) return PyLong_FromLong(st);
  PyObject* q_obj;
  PyObject* sc_obj = codes_tuple_items(op, c.q, c.sc, M, &q_obj);
  return Py_BuildValue("(NN)", q_obj, sc_obj);
}

PyObject* qk_impl(PyObject* const* a) {
  const int op = (int)PyLong_AsLong(a[0]);
  void* fn = PyLong_AsVoidPtr(a[1]);
  const at::Tensor& qg = *tensor_arg(a[2], "qg", false);
  const at::Tensor& k = *tensor_arg(a[3], "k", false);
  const at::Tensor& q_w = *tensor_arg(a[4], "q_w", false);
  const at::Tensor& k_w = *tensor_arg(a[5], "k_w", false);
  const int64_t Hq = PyLong_AsLongLong(a[6]), Hk = PyLong_AsLongLong(a[7]), D = PyLong_AsLongLong(a[8]);
  const float eps = (float)PyFloat_AsDouble(a[9]);
  const at::Tensor* given[5];
  const char* names[5] = {"q_out", "q_scale_out", "k_out", "k_scale_out", "gate_out"};
  for (int i = 0; i < 5; ++i) given[i] = tensor_arg(a[10 + i], names[i], true);
  if (PyErr_Occurred()) return nullptr;

  const c10::ScalarType bf = at::kBFloat16;
  const int64_t ld_qg = row_stride(qg, "qg", &bf), ld_k = row_stride(k, "k", &bf);
  const int64_t T = qg.size(0);
  if (k.size(0) != T) throw Refused{"qg and k must have the same number of tokens"};
  // The library sees row strides, not widths: a narrower view of a wider
  // buffer would pass its stride check and be read past its last column.
  int64_t hq_d = 0, wq = 0, wk = 0;
  if (Hq > 0 && Hk > 0 && D > 0 && !__builtin_mul_overflow(Hq, D, &hq_d) && !__builtin_mul_overflow(hq_d, 2, &wq) &&
      !__builtin_mul_overflow(Hk, D, &wk) && (qg.size(1) < wq || k.size(1) < wk))
    throw Refused{"qg must have at least 2 * num_q_heads * head_dim columns (" + std::to_string(wq) + ") and k " +
                  "num_k_heads * head_dim (" + std::to_string(wk) + ")"};
  for (const auto& [name, t] : {std::pair<const char*, const at::Tensor*>{"q_w", &q_w}, {"k_w", &k_w}}) {
    if (t->dim() != 1 || t->size(0) != D || t->scalar_type() != bf || !t->is_contiguous())
      throw Refused{std::string(name) + " must be a contiguous [head_dim] bfloat16 tensor"};
  }
  const c10::Device dev = qg.device();
  same_device(&k, "k", dev);
  same_device(&q_w, "q_w", dev);
  same_device(&k_w, "k_w", dev);
  const auto opt = qg.options();

  at::Tensor out[5];  // q, q_scale, k, k_scale, gate
  if (op == kQkBf16) {
    const int64_t heads[3] = {Hq, Hk, Hq};
    const int slot[3] = {0, 2, 4};
    for (int i = 0; i < 3; ++i) {
      const at::Tensor* t = given[slot[i]];
      out[slot[i]] = t != nullptr ? *t : at::empty({T, heads[i], D}, opt);
      const at::Tensor& o = out[slot[i]];
      if (o.dim() != 3 || o.size(0) != T || o.size(1) != heads[i] || o.size(2) != D || o.scalar_type() != bf ||
          !o.is_contiguous())
        throw Refused{std::string(names[slot[i]]) + " must be a contiguous [T, heads, head_dim] bfloat16 tensor"};
    }
    for (int i : {0, 2, 4}) same_device(&out[i], names[i], dev);
  } else if (op == kQkFp8) {
    const std::initializer_list<c10::ScalarType> codes = {at::kFloat8_e4m3fn, at::kByte};
    const std::initializer_list<c10::ScalarType> f32 = {at::kFloat};
    const std::initializer_list<c10::ScalarType> gate = {at::kBFloat16};
    const std::vector<int64_t> shapes[5] = {{T, Hq, D}, {T, Hq}, {T, Hk, D}, {T, Hk}, {T, Hq, D}};
    const std::initializer_list<c10::ScalarType>* dts[5] = {&codes, &f32, &codes, &f32, &gate};
    for (int i = 0; i < 5; ++i) {
      out[i] = given[i] != nullptr ? *given[i] : at::empty(shapes[i], opt.dtype(*dts[i]->begin()));
      const at::Tensor& o = out[i];
      const bool dt_ok = std::find(dts[i]->begin(), dts[i]->end(), o.scalar_type()) != dts[i]->end();
      if (o.sizes() != at::IntArrayRef(shapes[i]) || !dt_ok || !o.is_contiguous())
        throw Refused{std::string(names[i]) + " must be a contiguous " + shape_str(shapes[i]) + " tensor of " +
                      dtype_name(*dts[i]->begin())};
    }
    for (int i = 0; i < 5; ++i) same_device(&out[i], names[i], dev);
  } else if (op == kQkMxfp4) {
    const int64_t nb = std::max<int64_t>(floordiv(D, 32), 1);
    const std::vector<int64_t> shapes[5] = {{T, Hq, floordiv(D, 2)}, {T, Hq, nb}, {T, Hk, floordiv(D, 2)}, {T, Hk, nb},
                                            {T, Hq, D}};
    for (int i = 0; i < 5; ++i) {
      const c10::ScalarType odt = i == 4 ? at::kBFloat16 : at::kByte;
      out[i] = given[i] != nullptr ? checked_out(*given[i], shapes[i], {odt}, names[i], dev)
                                   : at::empty(shapes[i], opt.dtype(odt));
    }
  } else {
    PyErr_SetString(PyExc_ValueError, "qk: unknown operation");
    return nullptr;
  }

  const c10::DeviceGuard on_device(dev);
  void* stream = stream_of(a[15], dev);
  const void *qgp = qg.data_ptr(), *kp = k.data_ptr(), *qwp = q_w.data_ptr(), *kwp = k_w.data_ptr();
  int st;
  if (op == kQkBf16) {
    st = reinterpret_cast<QkFn>(fn)(qgp, ld_qg, kp, ld_k, qwp, kwp, T, Hq, Hk, D, eps, out[0].data_ptr(),
                                     out[2].data_ptr(), out[4].data_ptr(), stream);
  } else {
    st = reinterpret_cast<QkQuantFn>(fn)(qgp, ld_qg, kp, ld_k, qwp, kwp, T, Hq, Hk, D, eps, out[0].data_ptr(),
                                          out[1].data_ptr(), out[2].data_ptr(), out[3].data_ptr(), out[4].data_ptr(),
                                          stream);
  }
  if (st != 0) return PyLong_FromLong(st);
  if (op == kQkBf16) return Py_BuildValue("(NNN)", wrap(out[0]), wrap(out[2]), wrap(out[4]));
  return Py_BuildValue("(NNNNN)", wrap(out[0]), wrap(out[1]), wrap(out[2]), wrap(out[3]), wrap(out[4]));
}

// Refused arguments raise ValueError; an error from torch (an allocation that
// fails, say) raises RuntimeError.
template <PyObject* (*Impl)(PyObject* const*), Py_ssize_t kArgs>
PyObject* entry(PyObject*, PyObject* const* args, Py_ssize_t n) {
  if (n != kArgs) {
    PyErr_Format(PyExc_TypeError, "expected %zd arguments, got %zd", kArgs, n);
    return nullptr;
  }
  try {
    return Impl(args);
  } catch (const Refused& e) {
    PyErr_SetString(PyExc_ValueError, e.msg.c_str());
  } catch (const std::exception& e) {
    PyErr_SetString(PyExc_RuntimeError, e.what());
  }
  return nullptr;
}

PyMethodDef kMethods[] = {
    {"rows", reinterpret_cast<PyCFunction>(reinterpret_cast<void (*)(void)>(&entry<rows_impl, 13>)), METH_FASTCALL,
     "rows(op, (entry_bf16, entry_f16), x, residual, weight, eps, group, residual_out, q_out, scale_out, emit_y, "
     "y_out, stream) -> outputs tuple, or the status code"},
    {"quantize", reinterpret_cast<PyCFunction>(reinterpret_cast<void (*)(void)>(&entry<quantize_impl, 7>)),
     METH_FASTCALL, "quantize(op, (entry_bf16, entry_f16), y, group, q_out, scale_out, stream) -> (codes, scales), "
     "or the status code"},
    {"qk", reinterpret_cast<PyCFunction>(reinterpret_cast<void (*)(void)>(&entry<qk_impl, 16>)), METH_FASTCALL,
     "qk(op, entry, qg, k, q_w, k_w, Hq, Hk, D, eps, q_out, q_scale_out, k_out, k_scale_out, gate_out, stream) "
     "-> outputs tuple, or the status code"},
    {nullptr, nullptr, 0, nullptr}};

PyModuleDef kModule = {PyModuleDef_HEAD_INIT, "_marshal", "Argument marshalling of the library's entry points.", -1,
                       kMethods};

}  // namespace

PyMODINIT_FUNC PyInit__marshal() { return PyModule_Create(&kModule); }
