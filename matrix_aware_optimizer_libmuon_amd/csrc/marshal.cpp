// Argument marshalling of the Python binding.  No arithmetic of the method.
//
// Fills the C-ABI descriptor arrays of include/muon.h (muon_matrix_t,
// muon_ortho_t, muon_adamw_tensor_t) from lists of torch tensors, with the
// binding's checks: GPU tensors on one device, contiguous, 2-D where the call
// needs matrices, the element types each call accepts, matching shapes.  It
// lives in C++ because a grouped call over thousands of tensors would
// otherwise spend milliseconds of Python attribute access per step, longer
// than the GPU takes for the step itself.
//
// Errors raise ValueError (structure) or TypeError (element type) naming the
// offending list entry; nothing is written to the GPU from here.
#include <torch/extension.h>

#include <cstdint>
#include <string>
#include <vector>

#include "muon.h"

namespace {

namespace py = pybind11;
using OptTensor = c10::optional<at::Tensor>;

[[noreturn]] void fail_value(const char* list, size_t i, const std::string& what) {
  throw py::value_error(std::string(list) + "[" + std::to_string(i) + "] " + what);
}

[[noreturn]] void fail_type(const char* list, size_t i, const std::string& what) {
  throw py::type_error(std::string(list) + "[" + std::to_string(i) + "] " + what);
}

std::string shape_str(const at::Tensor& t) {
  std::string s = "(";
  for (int64_t d = 0; d < t.dim(); ++d) s += (d ? ", " : "") + std::to_string(t.size(d));
  return s + ")";
}

// GPU, on `dev`, contiguous, and 2-D when `matrix`.
void check_tensor(const at::Tensor& t, const c10::Device& dev, const char* list, size_t i,
                  bool matrix) {
  if (matrix && t.dim() != 2) fail_value(list, i, "must be 2-D, got shape " + shape_str(t));
  if (!t.is_contiguous()) fail_value(list, i, "must be contiguous");
  if (!t.is_cuda()) fail_value(list, i, "must be a GPU tensor");
  if (t.device() != dev) fail_value(list, i, "is on another device than params[0]");
}

void check_fp32(const at::Tensor& t, const char* list, size_t i) {
  if (t.scalar_type() != at::kFloat) fail_type(list, i, "must be float32");
}

int32_t elem_code(const at::Tensor& t, const char* list, size_t i) {
  if (t.scalar_type() == at::kFloat) return MUON_F32;
  if (t.scalar_type() == at::kBFloat16) return MUON_BF16;
  fail_type(list, i, "must be float32 or bfloat16");
}

void* ptr(const at::Tensor& t) { return t.data_ptr(); }

// muon_matrix_t[n] at `out`: params and momenta fp32 2-D, grads fp32/bf16 or
// None (skipped matrix), scales empty or one per matrix (<= 0: call level).
void fill_matrices(const std::vector<at::Tensor>& params, const std::vector<OptTensor>& grads,
                   const std::vector<at::Tensor>& moms, const std::vector<double>& scales,
                   uintptr_t out) {
  const size_t n = params.size();
  if (grads.size() != n || moms.size() != n)
    throw py::value_error("params, grads and moms must have the same length");
  if (!scales.empty() && scales.size() != n)
    throw py::value_error("scales must have one entry per matrix");
  auto* m = reinterpret_cast<muon_matrix_t*>(out);
  if (n == 0) return;
  const c10::Device dev = params[0].device();
  for (size_t i = 0; i < n; ++i) {
    const at::Tensor& p = params[i];
    const at::Tensor& mo = moms[i];
    check_tensor(p, dev, "params", i, true);
    check_fp32(p, "params", i);
    check_tensor(mo, dev, "moms", i, true);
    check_fp32(mo, "moms", i);
    if (mo.sizes() != p.sizes())
      fail_value("moms", i, "shape " + shape_str(mo) + " != param shape " + shape_str(p));
    muon_matrix_t& d = m[i];
    d.param = static_cast<float*>(ptr(p));
    d.momentum = static_cast<float*>(ptr(mo));
    d.rows = p.size(0);
    d.cols = p.size(1);
    d.scale = scales.empty() ? 0.0f : static_cast<float>(scales[i]);
    d.grad = nullptr;
    d.grad_dtype = MUON_F32;
    if (grads[i].has_value()) {
      const at::Tensor& g = *grads[i];
      check_tensor(g, dev, "grads", i, true);
      if (g.sizes() != p.sizes())
        fail_value("grads", i, "shape " + shape_str(g) + " != param shape " + shape_str(p));
      d.grad_dtype = elem_code(g, "grads", i);
      d.grad = ptr(g);
    }
  }
}

// muon_ortho_t[n] at `out`: inputs fp32/bf16 2-D, outputs bf16 of the same shape.
void fill_ortho(const std::vector<at::Tensor>& inputs, const std::vector<at::Tensor>& outputs,
                uintptr_t out) {
  const size_t n = inputs.size();
  if (outputs.size() != n) throw py::value_error("inputs and outputs must have the same length");
  auto* m = reinterpret_cast<muon_ortho_t*>(out);
  if (n == 0) return;
  const c10::Device dev = inputs[0].device();
  for (size_t i = 0; i < n; ++i) {
    const at::Tensor& x = inputs[i];
    const at::Tensor& y = outputs[i];
    check_tensor(x, dev, "inputs", i, true);
    check_tensor(y, dev, "outputs", i, true);
    if (y.scalar_type() != at::kBFloat16) fail_type("outputs", i, "must be bfloat16");
    if (y.sizes() != x.sizes()) fail_value("outputs", i, "shape mismatch");
    m[i].in = ptr(x);
    m[i].out = ptr(y);
    m[i].rows = x.size(0);
    m[i].cols = x.size(1);
    m[i].in_dtype = elem_code(x, "inputs", i);
  }
}

// muon_adamw_tensor_t[n] at `out`: any shape; param and moments fp32, grads
// fp32/bf16 shaped like the param or None; steps[i] >= 1 is checked by the
// library.
void fill_adamw(const std::vector<at::Tensor>& params, const std::vector<OptTensor>& grads,
                const std::vector<at::Tensor>& exp_avgs, const std::vector<at::Tensor>& exp_avg_sqs,
                const std::vector<int64_t>& steps, uintptr_t out) {
  const size_t n = params.size();
  if (grads.size() != n || exp_avgs.size() != n || exp_avg_sqs.size() != n || steps.size() != n)
    throw py::value_error(
        "params, grads, exp_avgs, exp_avg_sqs and steps must have the same length");
  auto* m = reinterpret_cast<muon_adamw_tensor_t*>(out);
  if (n == 0) return;
  const c10::Device dev = params[0].device();
  for (size_t i = 0; i < n; ++i) {
    const at::Tensor& p = params[i];
    check_tensor(p, dev, "params", i, false);
    check_fp32(p, "params", i);
    check_tensor(exp_avgs[i], dev, "exp_avgs", i, false);
    check_fp32(exp_avgs[i], "exp_avgs", i);
    check_tensor(exp_avg_sqs[i], dev, "exp_avg_sqs", i, false);
    check_fp32(exp_avg_sqs[i], "exp_avg_sqs", i);
    if (exp_avgs[i].sizes() != p.sizes() || exp_avg_sqs[i].sizes() != p.sizes())
      fail_value("params", i, "moment shapes differ from the param's");
    muon_adamw_tensor_t& d = m[i];
    d.param = static_cast<float*>(ptr(p));
    d.exp_avg = static_cast<float*>(ptr(exp_avgs[i]));
    d.exp_avg_sq = static_cast<float*>(ptr(exp_avg_sqs[i]));
    d.numel = p.numel();
    d.step = steps[i];
    d.grad = nullptr;
    d.grad_dtype = MUON_F32;
    d.reserved = 0;
    if (grads[i].has_value()) {
      const at::Tensor& g = *grads[i];
      check_tensor(g, dev, "grads", i, false);
      if (g.sizes() != p.sizes()) fail_value("grads", i, "must be shaped like its param");
      d.grad_dtype = elem_code(g, "grads", i);
      d.grad = ptr(g);
    }
  }
}

}  // namespace

PYBIND11_MODULE(_marshal, mod) {
  mod.doc() = "libmuon argument marshalling (fills C-ABI descriptor arrays from tensors)";
  mod.def("fill_matrices", &fill_matrices);
  mod.def("fill_ortho", &fill_ortho);
  mod.def("fill_adamw", &fill_adamw);
  mod.attr("MATRIX_BYTES") = sizeof(muon_matrix_t);
  mod.attr("ORTHO_BYTES") = sizeof(muon_ortho_t);
  mod.attr("ADAMW_BYTES") = sizeof(muon_adamw_tensor_t);
}
