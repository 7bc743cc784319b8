// Placeholder: path not built yet (supported() is false, so it is never chosen).
#include "gconv_internal.h"

namespace gconv {
namespace smallg {
bool supported(const Problem &) { return false; }
gconv_plan plan(const Problem &) { return gconv_plan{}; }
hipError_t launch(const Problem &, const Args &, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace smallg
}  // namespace gconv
