// placeholder until the MFMA backward lands
#include "internal.h"
