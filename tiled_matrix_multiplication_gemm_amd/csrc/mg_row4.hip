// Kernels of table row 4 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW(4, Cfg4, Fast4)
